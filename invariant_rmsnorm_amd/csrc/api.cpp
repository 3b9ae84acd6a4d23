// C-ABI entry points of librmsnorm_mi355x.so: argument checks on the host,
// then the gfx950 kernels (fwd.hip, bwd.hip). The declarations and their
// contract live in include/rmsnorm_mi355x.h.
//
// Every check runs before anything is enqueued, so a rejected call writes
// nothing. Unsupported input is reported, never routed to another code path
// (TransformerEngine issue "Expose Batch Invariant Kernels", checks table:
// unsupported combinations are rejected rather than silently falling back).
#include "rmsnorm_mi355x.h"

#include <cmath>
#include <cstdint>

#include "geometry.hpp"
#include "launch.hpp"
#include "plan.hpp"
#include "scratch.hpp"

namespace {

using rmsn::kMaxD;
static_assert(RMSN_NOALLOC_SCRATCH_BYTES == rmsn::kScratchBytes, "scratch size in the header");
// Row strides up to 2^24 elements keep every per-lane byte offset of a
// 64-row group below 2^31 (the kernels address rows through 32-bit offsets).
constexpr int64_t kMaxLd = int64_t{1} << 24;

struct Range {
  uintptr_t lo = 0, hi = 0;  // [lo, hi); empty when lo == hi
};

Range mat_range(const void* p, int64_t T, int64_t ld, int64_t D, int64_t elem) {
  if (p == nullptr || T <= 0) return {};
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return {lo, lo + static_cast<uintptr_t>(((T - 1) * ld + D) * elem)};
}

Range vec_range(const void* p, int64_t n, int64_t elem) {
  if (p == nullptr || n <= 0) return {};
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return {lo, lo + static_cast<uintptr_t>(n * elem)};
}

bool overlap(const Range& a, const Range& b) {
  return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

// Each output must be disjoint from every input and every other output.
template <size_t NO, size_t NI>
bool any_alias(const Range (&outs)[NO], const Range (&ins)[NI]) {
  for (size_t i = 0; i < NO; ++i) {
    for (size_t j = 0; j < NI; ++j)
      if (overlap(outs[i], ins[j])) return true;
    for (size_t j = i + 1; j < NO; ++j)
      if (overlap(outs[i], outs[j])) return true;
  }
  return false;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Row length: 1..32768.
rmsn_status check_D(int64_t D) {
  if (D <= 0) return RMSN_ERR_SHAPE;
  if (D > kMaxD) return RMSN_ERR_UNSUPPORTED_D;
  return RMSN_OK;
}

// A bf16 / fp16 [T, D] operand with row stride ld: shape, then (when T > 0)
// the pointer and its alignment. Rows of a multiple of 8 elements move as
// 16-byte vectors and need a 16-byte-aligned base and a stride of a
// multiple of 8; other rows move element by element and need 2-byte
// alignment only. T * ld is bounded by 2^60 elements, so every byte count
// the checks below form (an operand's extent, T floats of rstd) stays
// below 2^62.
constexpr int64_t kMaxElems = int64_t{1} << 60;
rmsn_status check_mat(const uint16_t* p, int64_t ld, int64_t T, int64_t D, bool required) {
  if (!required && p == nullptr) return RMSN_OK;
  if (ld < D || ld > kMaxLd) return RMSN_ERR_SHAPE;
  if (T > 0 && ld > kMaxElems / T) return RMSN_ERR_SHAPE;
  if (T == 0) return RMSN_OK;
  if (p == nullptr) return RMSN_ERR_NULL;
  if (D % 8 == 0 ? (!aligned(p, 16) || (ld % 8) != 0) : !aligned(p, 2)) return RMSN_ERR_MISALIGNED;
  return RMSN_OK;
}

rmsn_status check_f32(const float* p, uintptr_t align, bool required) {
  if (p == nullptr) return required ? RMSN_ERR_NULL : RMSN_OK;
  return aligned(p, align) ? RMSN_OK : RMSN_ERR_MISALIGNED;
}

#define RMSN_TRY(expr)                   \
  do {                                   \
    const rmsn_status s_ = (expr);       \
    if (s_ != RMSN_OK) return s_;        \
  } while (0)

rmsn_status hip_status(int rc) { return rc == 0 ? RMSN_OK : RMSN_ERR_HIP; }

// The forward reads its inputs with the streaming hint when x is well past
// the Infinity Cache (RMSN_STREAM_BYTES): the backward would find little of
// them there.
#ifndef RMSN_FWD_STREAM_X
#define RMSN_FWD_STREAM_X 1
#endif
// Bytes of x past which both kernels read it with the streaming hint: twice
// the Infinity Cache. Below that, keeping x's lines pays although x does
// not fit: the backward still finds part of it (measured, T x 4096 bf16,
// step with the cache flushed before it, never streaming / streaming past
// 256 MiB: x = 288 MiB 72.4 / 67.6%, 384 MiB 72.9 / 70.7%, 512 MiB
// 72.3 / 71.2%, 1 GiB 70.2 / 72.1%).
#ifndef RMSN_STREAM_BYTES
#define RMSN_STREAM_BYTES (2 * rmsn::kCacheBytes)
#endif
bool streams_x(int64_t T, int64_t D) { return T * D * 2 > static_cast<int64_t>(RMSN_STREAM_BYTES); }
int fwd_stream(int64_t T, int64_t D) { return RMSN_FWD_STREAM_X && streams_x(T, D); }

// Storage types of one call: activations (bf16 or fp16) and weights (bf16,
// fp16 or fp32). The entry points without a _dt suffix use bf16 / fp32.
struct Types {
  int dt = RMSN_DTYPE_BF16;
  int wdt = RMSN_DTYPE_F32;
};
bool bad_types(const Types& t) {
  return (t.dt != RMSN_DTYPE_BF16 && t.dt != RMSN_DTYPE_F16) ||
         (t.wdt != RMSN_DTYPE_BF16 && t.wdt != RMSN_DTYPE_F16 && t.wdt != RMSN_DTYPE_F32);
}
int64_t weight_bytes(const Types& t) { return t.wdt == RMSN_DTYPE_F32 ? 4 : 2; }

rmsn_status check_ptr(const void* p, uintptr_t align, bool required) {
  if (p == nullptr) return required ? RMSN_ERR_NULL : RMSN_OK;
  return aligned(p, align) ? RMSN_OK : RMSN_ERR_MISALIGNED;
}

bool bad_activation(int act) { return act != RMSN_GATE_SILU && act != RMSN_GATE_SIGMOID; }

rmsn_status fwd_common(const uint16_t* x, int64_t ld_x, const uint16_t* z, int64_t ld_z,
                       bool gated, int act, int rounding, const void* gamma, int zc, float eps,
                       int64_t T, int64_t D, uint16_t* y, int64_t ld_y, uint16_t* res,
                       int64_t ld_res, bool residual, float* rstd, void* stream,
                       Types ty = Types{}) {
  if (bad_types(ty)) return RMSN_ERR_MODE;
  if (gated && (bad_activation(act) ||
                (rounding != RMSN_GATED_ROUND_FP32 && rounding != RMSN_GATED_ROUND_CAST)))
    return RMSN_ERR_MODE;
  if (T < 0) return RMSN_ERR_SHAPE;
  RMSN_TRY(check_D(D));
  RMSN_TRY(check_mat(x, ld_x, T, D, true));
  if (gated) RMSN_TRY(check_mat(z, ld_z, T, D, true));
  RMSN_TRY(check_mat(y, ld_y, T, D, true));
  if (residual) RMSN_TRY(check_mat(res, ld_res, T, D, true));
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return RMSN_ERR_EPS;
  if (T == 0) return RMSN_OK;
  RMSN_TRY(check_ptr(gamma, 16, true));
  RMSN_TRY(check_f32(rstd, 4, false));
  const Range outs[] = {mat_range(y, T, ld_y, D, 2), mat_range(res, T, ld_res, D, 2),
                        vec_range(rstd, T, 4)};
  const Range ins[] = {mat_range(x, T, ld_x, D, 2), mat_range(z, T, ld_z, D, 2),
                       vec_range(gamma, D, weight_bytes(ty))};
  if (any_alias(outs, ins)) return RMSN_ERR_ALIASING;

  rmsn::FwdArgs a{x, ld_x, gated ? z : nullptr, ld_z, act, rounding == RMSN_GATED_ROUND_CAST,
                  gamma, ty.wdt, ty.dt, zc != 0, eps, T, static_cast<int>(D), y, ld_y,
                  residual ? res : nullptr, ld_res, rstd, nullptr, 0, fwd_stream(T, D)};
  return hip_status(rmsn::launch_fwd(a, stream));
}

// Aliasing of the fused add forward: y may be x itself and residual_out the
// residual input itself (the same memory and row stride: each lane stores
// only values it computed from elements it has already loaded at those
// addresses, and rows do not overlap); any other overlap is rejected.
bool add_fwd_alias(const uint16_t* x, int64_t ld_x, const uint16_t* rin, int64_t ld_rin,
                   const void* gamma, int64_t gamma_elem, int64_t T, int64_t D, const uint16_t* y,
                   int64_t ld_y, const uint16_t* rout, int64_t ld_rout, const float* rstd) {
  const Range X = mat_range(x, T, ld_x, D, 2), RI = mat_range(rin, T, ld_rin, D, 2),
              G = vec_range(gamma, D, gamma_elem), Y = mat_range(y, T, ld_y, D, 2),
              RO = mat_range(rout, T, ld_rout, D, 2), RS = vec_range(rstd, T, 4);
  const bool y_in_place = y == x && ld_y == ld_x;
  const bool r_in_place = rout == rin && ld_rout == ld_rin;
  if ((!y_in_place && overlap(Y, X)) || overlap(Y, RI) || overlap(Y, G)) return true;
  if ((!r_in_place && overlap(RO, RI)) || overlap(RO, X) || overlap(RO, G)) return true;
  if (overlap(RS, X) || overlap(RS, RI) || overlap(RS, G)) return true;
  return overlap(Y, RO) || overlap(Y, RS) || overlap(RO, RS);
}

size_t workspace_bytes(int64_t T, int64_t D) {
  if (T <= 0 || check_D(D) != RMSN_OK) return 0;
  const rmsn::BwdPlan p = rmsn::bwd_plan(T, D);
  return static_cast<size_t>(p.chunks) * static_cast<size_t>(rmsn::part_stride(D)) * sizeof(float);
}

// The gate operands of the gated backward (absent for the other forms).
struct GateIO {
  const uint16_t* z = nullptr;
  int64_t ld_z = 0;
  uint16_t* dz = nullptr;
  int64_t ld_dz = 0;
};

// Checks shared by the backward entry points; `dgamma` is only checked for
// aliasing here (rmsnorm_bwd_rows passes nullptr).
rmsn_status check_bwd(const uint16_t* g, int64_t ld_g, const uint16_t* x, int64_t ld_x,
                      const float* rstd, const void* gamma, int64_t T, int64_t D,
                      const uint16_t* gres, int64_t ld_gres, uint16_t* dx, int64_t ld_dx,
                      bool want_part, const float* dgamma, void* ws, size_t ws_bytes,
                      bool gated = false, const GateIO& gate = GateIO{},
                      const uint16_t* rin = nullptr, int64_t ld_rin = 0, bool add = false,
                      Types ty = Types{}) {
  if (bad_types(ty)) return RMSN_ERR_MODE;
  if (T < 0) return RMSN_ERR_SHAPE;
  RMSN_TRY(check_D(D));
  RMSN_TRY(check_mat(g, ld_g, T, D, true));
  RMSN_TRY(check_mat(x, ld_x, T, D, true));
  if (add) RMSN_TRY(check_mat(rin, ld_rin, T, D, true));
  RMSN_TRY(check_mat(gres, ld_gres, T, D, false));
  RMSN_TRY(check_mat(dx, ld_dx, T, D, false));
  if (gated) {
    RMSN_TRY(check_mat(gate.z, gate.ld_z, T, D, true));
    RMSN_TRY(check_mat(gate.dz, gate.ld_dz, T, D, false));
  }
  if (T == 0) return RMSN_OK;
  RMSN_TRY(check_f32(rstd, 4, true));
  // The rows kernel loads the weights whatever it writes, so gamma is
  // required even for a weight-gradient-only call.
  RMSN_TRY(check_ptr(gamma, 16, true));
  if (want_part) {
    if (ws == nullptr || ws_bytes < workspace_bytes(T, D)) return RMSN_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return RMSN_ERR_MISALIGNED;
  }
  const Range outs[] = {mat_range(dx, T, ld_dx, D, 2),
                        want_part ? vec_range(ws, static_cast<int64_t>(workspace_bytes(T, D)), 1)
                                  : Range{},
                        vec_range(dgamma, D, 4), mat_range(gate.dz, T, gate.ld_dz, D, 2)};
  const Range ins[] = {mat_range(g, T, ld_g, D, 2), mat_range(x, T, ld_x, D, 2),
                       vec_range(rstd, T, 4), vec_range(gamma, D, weight_bytes(ty)),
                       mat_range(gres, T, ld_gres, D, 2), mat_range(gate.z, T, gate.ld_z, D, 2),
                       mat_range(add ? rin : nullptr, T, ld_rin, D, 2)};
  if (any_alias(outs, ins)) return RMSN_ERR_ALIASING;
  return RMSN_OK;
}

rmsn::BwdArgs bwd_args(const uint16_t* g, int64_t ld_g, const uint16_t* x, int64_t ld_x,
                       const float* rstd, const void* gamma, int zc, int64_t T, int64_t D,
                       const uint16_t* gres, int64_t ld_gres, uint16_t* dx, int64_t ld_dx,
                       void* ws, const GateIO& gate = GateIO{}, int act = 0,
                       const uint16_t* rin = nullptr, int64_t ld_rin = 0, Types ty = Types{}) {
  const rmsn::BwdPlan p = rmsn::bwd_plan(T, D);
  return rmsn::BwdArgs{g, ld_g, x, ld_x, rstd, gamma, ty.wdt, ty.dt, zc != 0, T, static_cast<int>(D),
                       dx ? gres : nullptr, ld_gres, dx, ld_dx, static_cast<float*>(ws),
                       p.chunks, p.group_blocks, gate.z, gate.ld_z, act, gate.dz, gate.ld_dz,
                       streams_x(T, D), rin, ld_rin};
}

// dgamma from the workspace partials (zeros when T == 0).
rmsn_status finish_dgamma(void* workspace, int64_t T, int64_t D, float* dgamma, void* stream) {
  const int64_t chunks = T > 0 ? rmsn::bwd_plan(T, D).chunks : 0;
  return hip_status(rmsn::launch_bwd_finish(static_cast<const float*>(workspace), chunks,
                                            static_cast<int>(D), dgamma, stream));
}

// The _dt entry points pass 16-bit activations as untyped pointers.
const uint16_t* u16(const void* p) { return static_cast<const uint16_t*>(p); }
uint16_t* u16(void* p) { return static_cast<uint16_t*>(p); }

rmsn_status add_fwd_common(const uint16_t* x, int64_t ld_x, const uint16_t* residual,
                           int64_t ld_res, const void* gamma, int zc, float eps, int64_t T,
                           int64_t D, uint16_t* y, int64_t ld_y, uint16_t* residual_out,
                           int64_t ld_rout, float* rstd, void* stream, Types ty) {
  if (bad_types(ty)) return RMSN_ERR_MODE;
  if (T < 0) return RMSN_ERR_SHAPE;
  RMSN_TRY(check_D(D));
  RMSN_TRY(check_mat(x, ld_x, T, D, true));
  RMSN_TRY(check_mat(residual, ld_res, T, D, true));
  RMSN_TRY(check_mat(y, ld_y, T, D, true));
  RMSN_TRY(check_mat(residual_out, ld_rout, T, D, true));
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return RMSN_ERR_EPS;
  if (T == 0) return RMSN_OK;
  RMSN_TRY(check_ptr(gamma, 16, true));
  RMSN_TRY(check_f32(rstd, 4, false));
  if (add_fwd_alias(x, ld_x, residual, ld_res, gamma, weight_bytes(ty), T, D, y, ld_y,
                    residual_out, ld_rout, rstd))
    return RMSN_ERR_ALIASING;
  const rmsn::FwdArgs a{x, ld_x, nullptr, 0, 0, 0, gamma, ty.wdt, ty.dt, zc != 0, eps, T,
                        static_cast<int>(D), y, ld_y, residual_out, ld_rout, rstd, residual,
                        ld_res, fwd_stream(T, D)};
  return hip_status(rmsn::launch_fwd(a, stream));
}

rmsn_status gated_bwd_common(const uint16_t* g, int64_t ld_g, const uint16_t* x, int64_t ld_x,
                             const uint16_t* z, int64_t ld_z, const float* rstd,
                             const void* gamma, int zc, int64_t T, int64_t D, int activation,
                             uint16_t* dx, int64_t ld_dx, uint16_t* dz, int64_t ld_dz,
                             float* dgamma, void* workspace, size_t ws_bytes, void* stream,
                             Types ty) {
  if (bad_types(ty) || bad_activation(activation)) return RMSN_ERR_MODE;
  if (dx == nullptr && dz == nullptr && dgamma == nullptr) return RMSN_ERR_NULL;
  if (dgamma != nullptr) RMSN_TRY(check_f32(dgamma, 16, true));
  const GateIO gate{z, ld_z, dz, ld_dz};
  RMSN_TRY(check_bwd(g, ld_g, x, ld_x, rstd, gamma, T, D, nullptr, 0, dx, ld_dx,
                     dgamma != nullptr, dgamma, workspace, ws_bytes, true, gate, nullptr, 0,
                     false, ty));
  if (T > 0) {
    const rmsn::BwdArgs a = bwd_args(g, ld_g, x, ld_x, rstd, gamma, zc, T, D, nullptr, 0, dx,
                                     ld_dx, dgamma != nullptr ? workspace : nullptr, gate,
                                     activation, nullptr, 0, ty);
    RMSN_TRY(hip_status(rmsn::launch_bwd_rows(a, stream)));
  }
  if (dgamma == nullptr) return RMSN_OK;
  return finish_dgamma(workspace, T, D, dgamma, stream);
}

// The fused add-norm backward: rows kernel (dh and/or the partials), then
// the finish kernel when dgamma is wanted.
rmsn_status add_bwd_common(const uint16_t* g, int64_t ld_g, const uint16_t* x, int64_t ld_x,
                           const uint16_t* residual, int64_t ld_res, const float* rstd,
                           const void* gamma, int zc, int64_t T, int64_t D,
                           const uint16_t* g_rout, int64_t ld_gro, uint16_t* dh, int64_t ld_dh,
                           float* dgamma, void* workspace, size_t ws_bytes, void* stream,
                           Types ty) {
  if (bad_types(ty)) return RMSN_ERR_MODE;
  if (dh == nullptr && dgamma == nullptr) return RMSN_ERR_NULL;
  if (dgamma != nullptr) RMSN_TRY(check_f32(dgamma, 16, true));
  RMSN_TRY(check_bwd(g, ld_g, x, ld_x, rstd, gamma, T, D, g_rout, ld_gro, dh, ld_dh,
                     dgamma != nullptr, dgamma, workspace, ws_bytes, false, GateIO{}, residual,
                     ld_res, true, ty));
  if (T > 0) {
    const rmsn::BwdArgs a = bwd_args(g, ld_g, x, ld_x, rstd, gamma, zc, T, D, g_rout, ld_gro, dh,
                                     ld_dh, dgamma != nullptr ? workspace : nullptr, GateIO{}, 0,
                                     residual, ld_res, ty);
    RMSN_TRY(hip_status(rmsn::launch_bwd_rows(a, stream)));
  }
  if (dgamma == nullptr) return RMSN_OK;
  return finish_dgamma(workspace, T, D, dgamma, stream);
}

}  // namespace

extern "C" {

int rmsnorm_abi_version(void) { return RMSN_ABI_VERSION; }

const char* rmsnorm_status_string(int status) {
  switch (status) {
    case RMSN_OK: return "RMSN_OK";
    case RMSN_ERR_NULL: return "RMSN_ERR_NULL: a required pointer is NULL";
    case RMSN_ERR_SHAPE: return "RMSN_ERR_SHAPE: T < 0, D <= 0, ld < D or ld > 2^24";
    case RMSN_ERR_UNSUPPORTED_D:
      return "RMSN_ERR_UNSUPPORTED_D: D must be in [1, 32768]; the GEMM's K a positive multiple "
             "of 32";
    case RMSN_ERR_MISALIGNED: return "RMSN_ERR_MISALIGNED: pointers and row strides must be 16-byte aligned";
    case RMSN_ERR_EPS: return "RMSN_ERR_EPS: eps must be finite and >= 0";
    case RMSN_ERR_ALIASING: return "RMSN_ERR_ALIASING: an output overlaps an input or another output";
    case RMSN_ERR_WORKSPACE: return "RMSN_ERR_WORKSPACE: workspace missing or too small";
    case RMSN_ERR_HIP: return "RMSN_ERR_HIP: the HIP runtime refused a kernel launch";
    case RMSN_ERR_MODE: return "RMSN_ERR_MODE: unknown gate activation, rounding convention or storage type";
    default: return "unknown rmsn_status";
  }
}

rmsn_status rmsnorm_fwd(const uint16_t* x, int64_t ld_x, const float* gamma, int zero_centered_gamma,
                        float eps, int64_t T, int64_t D, uint16_t* y, int64_t ld_y, float* rstd,
                        void* stream) {
  return fwd_common(x, ld_x, nullptr, 0, false, 0, 0, gamma, zero_centered_gamma, eps, T, D, y,
                    ld_y, nullptr, 0, false, rstd, stream);
}

rmsn_status rmsnorm_residual_fwd(const uint16_t* x, int64_t ld_x, const float* gamma,
                                 int zero_centered_gamma, float eps, int64_t T, int64_t D,
                                 uint16_t* y, int64_t ld_y, uint16_t* residual_out, int64_t ld_res,
                                 float* rstd, void* stream) {
  return fwd_common(x, ld_x, nullptr, 0, false, 0, 0, gamma, zero_centered_gamma, eps, T, D, y,
                    ld_y, residual_out, ld_res, true, rstd, stream);
}

rmsn_status rmsnorm_gated_fwd(const uint16_t* x, int64_t ld_x, const uint16_t* z, int64_t ld_z,
                              const float* gamma, int zero_centered_gamma, float eps, int64_t T,
                              int64_t D, uint16_t* out, int64_t ld_out, float* rstd, void* stream) {
  return fwd_common(x, ld_x, z, ld_z, true, RMSN_GATE_SILU, RMSN_GATED_ROUND_FP32, gamma,
                    zero_centered_gamma, eps, T, D, out, ld_out, nullptr, 0, false, rstd, stream);
}

rmsn_status rmsnorm_gated_fwd_ex(const uint16_t* x, int64_t ld_x, const uint16_t* z, int64_t ld_z,
                                 const float* gamma, int zero_centered_gamma, float eps, int64_t T,
                                 int64_t D, int activation, int rounding, uint16_t* out,
                                 int64_t ld_out, float* rstd, void* stream) {
  return fwd_common(x, ld_x, z, ld_z, true, activation, rounding, gamma, zero_centered_gamma, eps,
                    T, D, out, ld_out, nullptr, 0, false, rstd, stream);
}

size_t rmsnorm_bwd_workspace_bytes(int64_t T, int64_t D) { return workspace_bytes(T, D); }

rmsn_status rmsnorm_bwd_partials_layout(int64_t T, int64_t D, int64_t* block_rows,
                                        int64_t* group_blocks, int64_t* chunks) {
  if (T < 0) return RMSN_ERR_SHAPE;
  RMSN_TRY(check_D(D));
  const rmsn::BwdPlan p = rmsn::bwd_plan(T, D);
  if (block_rows) *block_rows = p.block_rows;
  if (group_blocks) *group_blocks = p.group_blocks;
  if (chunks) *chunks = p.chunks;
  return RMSN_OK;
}

int rmsnorm_dgamma_chunk_rows(int64_t D) {
  if (check_D(D) != RMSN_OK) return 0;
  return static_cast<int>(rmsn::bwd_rows_per_step(D));
}

rmsn_status rmsnorm_bwd_rows(const uint16_t* g, int64_t ld_g, const uint16_t* x, int64_t ld_x,
                             const float* rstd, const float* gamma, int zero_centered_gamma,
                             int64_t T, int64_t D, const uint16_t* g_residual, int64_t ld_gres,
                             uint16_t* dx, int64_t ld_dx, void* workspace, size_t workspace_bytes_,
                             void* stream) {
  if (dx == nullptr && workspace == nullptr) return RMSN_ERR_NULL;
  RMSN_TRY(check_bwd(g, ld_g, x, ld_x, rstd, gamma, T, D, g_residual, ld_gres, dx, ld_dx,
                     workspace != nullptr, nullptr, workspace, workspace_bytes_));
  if (T == 0) return RMSN_OK;
  const rmsn::BwdArgs a = bwd_args(g, ld_g, x, ld_x, rstd, gamma, zero_centered_gamma, T, D,
                                   g_residual, ld_gres, dx, ld_dx, workspace);
  return hip_status(rmsn::launch_bwd_rows(a, stream));
}

rmsn_status rmsnorm_bwd_finish(const void* workspace, size_t workspace_bytes_, int64_t T, int64_t D,
                               float* dgamma, void* stream) {
  if (T < 0) return RMSN_ERR_SHAPE;
  RMSN_TRY(check_D(D));
  RMSN_TRY(check_f32(dgamma, 16, true));
  const size_t need = workspace_bytes(T, D);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes_ < need) return RMSN_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return RMSN_ERR_MISALIGNED;
    const Range outs[] = {vec_range(dgamma, D, 4)};
    const Range ins[] = {vec_range(workspace, static_cast<int64_t>(need), 1)};
    if (any_alias(outs, ins)) return RMSN_ERR_ALIASING;
  }
  return finish_dgamma(const_cast<void*>(workspace), T, D, dgamma, stream);
}

rmsn_status rmsnorm_bwd(const uint16_t* g, int64_t ld_g, const uint16_t* x, int64_t ld_x,
                        const float* rstd, const float* gamma, int zero_centered_gamma, int64_t T,
                        int64_t D, const uint16_t* g_residual, int64_t ld_gres, uint16_t* dx,
                        int64_t ld_dx, float* dgamma, void* workspace, size_t workspace_bytes_,
                        void* stream) {
  if (dx == nullptr && dgamma == nullptr) return RMSN_ERR_NULL;
  if (dgamma != nullptr) RMSN_TRY(check_f32(dgamma, 16, true));
  RMSN_TRY(check_bwd(g, ld_g, x, ld_x, rstd, gamma, T, D, g_residual, ld_gres, dx, ld_dx,
                     dgamma != nullptr, dgamma, workspace, workspace_bytes_));
  if (T > 0) {
    const rmsn::BwdArgs a = bwd_args(g, ld_g, x, ld_x, rstd, gamma, zero_centered_gamma, T, D,
                                     g_residual, ld_gres, dx, ld_dx,
                                     dgamma != nullptr ? workspace : nullptr);
    RMSN_TRY(hip_status(rmsn::launch_bwd_rows(a, stream)));
  }
  if (dgamma == nullptr) return RMSN_OK;
  return finish_dgamma(workspace, T, D, dgamma, stream);
}

rmsn_status rmsnorm_bwd_noalloc(const uint16_t* g, int64_t ld_g, const uint16_t* x,
                                int64_t ld_x, const float* rstd, const float* gamma,
                                int zero_centered_gamma, int64_t T, int64_t D,
                                const uint16_t* g_residual, int64_t ld_gres, uint16_t* dx,
                                int64_t ld_dx, float* dgamma, void* stream) {
  if (dx == nullptr && dgamma == nullptr) return RMSN_ERR_NULL;
  if (dgamma != nullptr) RMSN_TRY(check_f32(dgamma, 16, true));
  // every argument but the workspace, as rmsnorm_bwd checks them
  RMSN_TRY(check_bwd(g, ld_g, x, ld_x, rstd, gamma, T, D, g_residual, ld_gres, dx, ld_dx, false,
                     dgamma, nullptr, 0));
  void* ws = nullptr;
  if (dgamma != nullptr && T > 0) {
    if (workspace_bytes(T, D) > rmsn::kScratchBytes) return RMSN_ERR_WORKSPACE;
    RMSN_TRY(hip_status(rmsn::scratch_ptr(&ws)));
  }
  if (T > 0) {
    const rmsn::BwdArgs a = bwd_args(g, ld_g, x, ld_x, rstd, gamma, zero_centered_gamma, T, D,
                                     g_residual, ld_gres, dx, ld_dx, ws);
    RMSN_TRY(hip_status(rmsn::launch_bwd_rows(a, stream)));
  }
  if (dgamma == nullptr) return RMSN_OK;
  return finish_dgamma(ws, T, D, dgamma, stream);
}

rmsn_status rmsnorm_gated_bwd(const uint16_t* g, int64_t ld_g, const uint16_t* x, int64_t ld_x,
                              const uint16_t* z, int64_t ld_z, const float* rstd,
                              const float* gamma, int zero_centered_gamma, int64_t T, int64_t D,
                              int activation, uint16_t* dx, int64_t ld_dx, uint16_t* dz,
                              int64_t ld_dz, float* dgamma, void* workspace,
                              size_t workspace_bytes_, void* stream) {
  return gated_bwd_common(g, ld_g, x, ld_x, z, ld_z, rstd, gamma, zero_centered_gamma, T, D,
                          activation, dx, ld_dx, dz, ld_dz, dgamma, workspace, workspace_bytes_,
                          stream, Types{});
}

rmsn_status rmsnorm_add_fwd(const uint16_t* x, int64_t ld_x, const uint16_t* residual,
                            int64_t ld_res, const float* gamma, int zero_centered_gamma, float eps,
                            int64_t T, int64_t D, uint16_t* y, int64_t ld_y, uint16_t* residual_out,
                            int64_t ld_rout, float* rstd, void* stream) {
  return add_fwd_common(x, ld_x, residual, ld_res, gamma, zero_centered_gamma, eps, T, D, y, ld_y,
                        residual_out, ld_rout, rstd, stream, Types{});
}

rmsn_status rmsnorm_add_bwd_rows(const uint16_t* g, int64_t ld_g, const uint16_t* x, int64_t ld_x,
                                 const uint16_t* residual, int64_t ld_res, const float* rstd,
                                 const float* gamma, int zero_centered_gamma, int64_t T, int64_t D,
                                 const uint16_t* g_residual_out, int64_t ld_gro, uint16_t* dh,
                                 int64_t ld_dh, void* workspace, size_t workspace_bytes_,
                                 void* stream) {
  if (dh == nullptr && workspace == nullptr) return RMSN_ERR_NULL;
  RMSN_TRY(check_bwd(g, ld_g, x, ld_x, rstd, gamma, T, D, g_residual_out, ld_gro, dh, ld_dh,
                     workspace != nullptr, nullptr, workspace, workspace_bytes_, false, GateIO{},
                     residual, ld_res, true));
  if (T == 0) return RMSN_OK;
  const rmsn::BwdArgs a = bwd_args(g, ld_g, x, ld_x, rstd, gamma, zero_centered_gamma, T, D,
                                   g_residual_out, ld_gro, dh, ld_dh, workspace, GateIO{}, 0,
                                   residual, ld_res);
  return hip_status(rmsn::launch_bwd_rows(a, stream));
}

rmsn_status rmsnorm_add_bwd(const uint16_t* g, int64_t ld_g, const uint16_t* x, int64_t ld_x,
                            const uint16_t* residual, int64_t ld_res, const float* rstd,
                            const float* gamma, int zero_centered_gamma, int64_t T, int64_t D,
                            const uint16_t* g_residual_out, int64_t ld_gro, uint16_t* dh,
                            int64_t ld_dh, float* dgamma, void* workspace, size_t workspace_bytes_,
                            void* stream) {
  return add_bwd_common(g, ld_g, x, ld_x, residual, ld_res, rstd, gamma, zero_centered_gamma, T, D,
                        g_residual_out, ld_gro, dh, ld_dh, dgamma, workspace, workspace_bytes_,
                        stream, Types{});
}

rmsn_status rmsnorm_fwd_dt(int act_dtype, int weight_dtype, const void* x, int64_t ld_x,
                           const void* gamma, int zero_centered_gamma, float eps, int64_t T,
                           int64_t D, void* y, int64_t ld_y, float* rstd, void* stream) {
  return fwd_common(static_cast<const uint16_t*>(x), ld_x, nullptr, 0, false, 0, 0, gamma,
                    zero_centered_gamma, eps, T, D, static_cast<uint16_t*>(y), ld_y, nullptr, 0,
                    false, rstd, stream, Types{act_dtype, weight_dtype});
}

rmsn_status rmsnorm_bwd_dt(int act_dtype, int weight_dtype, const void* g, int64_t ld_g,
                           const void* x, int64_t ld_x, const float* rstd, const void* gamma,
                           int zero_centered_gamma, int64_t T, int64_t D, const void* g_residual,
                           int64_t ld_gres, void* dx, int64_t ld_dx, float* dgamma,
                           void* workspace, size_t workspace_bytes_, void* stream) {
  const Types ty{act_dtype, weight_dtype};
  if (bad_types(ty)) return RMSN_ERR_MODE;
  if (dx == nullptr && dgamma == nullptr) return RMSN_ERR_NULL;
  if (dgamma != nullptr) RMSN_TRY(check_f32(dgamma, 16, true));
  const auto* g16 = static_cast<const uint16_t*>(g);
  const auto* x16 = static_cast<const uint16_t*>(x);
  const auto* gr16 = static_cast<const uint16_t*>(g_residual);
  auto* dx16 = static_cast<uint16_t*>(dx);
  RMSN_TRY(check_bwd(g16, ld_g, x16, ld_x, rstd, gamma, T, D, gr16, ld_gres, dx16, ld_dx,
                     dgamma != nullptr, dgamma, workspace, workspace_bytes_, false, GateIO{},
                     nullptr, 0, false, ty));
  if (T > 0) {
    const rmsn::BwdArgs a = bwd_args(g16, ld_g, x16, ld_x, rstd, gamma, zero_centered_gamma, T, D,
                                     gr16, ld_gres, dx16, ld_dx,
                                     dgamma != nullptr ? workspace : nullptr, GateIO{}, 0, nullptr,
                                     0, ty);
    RMSN_TRY(hip_status(rmsn::launch_bwd_rows(a, stream)));
  }
  if (dgamma == nullptr) return RMSN_OK;
  return finish_dgamma(workspace, T, D, dgamma, stream);
}

rmsn_status rmsnorm_gated_fwd_dt(int act_dtype, int weight_dtype, const void* x, int64_t ld_x,
                                 const void* z, int64_t ld_z, const void* gamma,
                                 int zero_centered_gamma, float eps, int64_t T, int64_t D,
                                 int activation, int rounding, void* out, int64_t ld_out,
                                 float* rstd, void* stream) {
  return fwd_common(u16(x), ld_x, u16(z), ld_z, true, activation, rounding, gamma,
                    zero_centered_gamma, eps, T, D, u16(out), ld_out, nullptr, 0, false, rstd,
                    stream, Types{act_dtype, weight_dtype});
}

rmsn_status rmsnorm_gated_bwd_dt(int act_dtype, int weight_dtype, const void* g, int64_t ld_g,
                                 const void* x, int64_t ld_x, const void* z, int64_t ld_z,
                                 const float* rstd, const void* gamma, int zero_centered_gamma,
                                 int64_t T, int64_t D, int activation, void* dx, int64_t ld_dx,
                                 void* dz, int64_t ld_dz, float* dgamma, void* workspace,
                                 size_t workspace_bytes_, void* stream) {
  return gated_bwd_common(u16(g), ld_g, u16(x), ld_x, u16(z), ld_z, rstd, gamma,
                          zero_centered_gamma, T, D, activation, u16(dx), ld_dx, u16(dz), ld_dz,
                          dgamma, workspace, workspace_bytes_, stream,
                          Types{act_dtype, weight_dtype});
}

rmsn_status rmsnorm_add_fwd_dt(int act_dtype, int weight_dtype, const void* x, int64_t ld_x,
                               const void* residual, int64_t ld_res, const void* gamma,
                               int zero_centered_gamma, float eps, int64_t T, int64_t D, void* y,
                               int64_t ld_y, void* residual_out, int64_t ld_rout, float* rstd,
                               void* stream) {
  return add_fwd_common(u16(x), ld_x, u16(residual), ld_res, gamma, zero_centered_gamma, eps, T,
                        D, u16(y), ld_y, u16(residual_out), ld_rout, rstd, stream,
                        Types{act_dtype, weight_dtype});
}

rmsn_status rmsnorm_add_bwd_dt(int act_dtype, int weight_dtype, const void* g, int64_t ld_g,
                               const void* x, int64_t ld_x, const void* residual, int64_t ld_res,
                               const float* rstd, const void* gamma, int zero_centered_gamma,
                               int64_t T, int64_t D, const void* g_residual_out, int64_t ld_gro,
                               void* dh, int64_t ld_dh, float* dgamma, void* workspace,
                               size_t workspace_bytes_, void* stream) {
  return add_bwd_common(u16(g), ld_g, u16(x), ld_x, u16(residual), ld_res, rstd, gamma,
                        zero_centered_gamma, T, D, u16(g_residual_out), ld_gro, u16(dh), ld_dh,
                        dgamma, workspace, workspace_bytes_, stream,
                        Types{act_dtype, weight_dtype});
}

rmsn_status bigemm_bf16_xwt(const uint16_t* x, int64_t ld_x, const uint16_t* w, int64_t ld_w,
                            int64_t M, int64_t N, int64_t K, uint16_t* y, int64_t ld_y,
                            void* stream) {
  if (M < 0 || N < 0 || K < 0) return RMSN_ERR_SHAPE;
  if (K == 0 || K % 32 != 0) return RMSN_ERR_UNSUPPORTED_D;
  constexpr int64_t kMaxGemmLd = int64_t{1} << 21;  // keeps 256-row byte counts below 2^30
  if (ld_x < K || ld_w < K || ld_y < N || ld_x > kMaxGemmLd || ld_w > kMaxGemmLd)
    return RMSN_ERR_SHAPE;
  // Y's extent (M - 1) * ld_y + N elements stays below 2^60, its bytes below 2^61
  if (M > 0 && ld_y > kMaxElems / M) return RMSN_ERR_SHAPE;
  if (M == 0 || N == 0) return RMSN_OK;
  // the launch grid has one workgroup per tile, at most 2^31 - 1
  if ((M + 31) / 32 > INT32_MAX / ((N + 63) / 64)) return RMSN_ERR_SHAPE;
  if (x == nullptr || w == nullptr || y == nullptr) return RMSN_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w, 16) || ld_x % 8 != 0 || ld_w % 8 != 0 || !aligned(y, 2))
    return RMSN_ERR_MISALIGNED;
  const Range outs[] = {mat_range(y, M, ld_y, N, 2)};
  const Range ins[] = {mat_range(x, M, ld_x, K, 2), mat_range(w, N, ld_w, K, 2)};
  if (any_alias(outs, ins)) return RMSN_ERR_ALIASING;
  const rmsn::GemmArgs a{x, ld_x, w, ld_w, M, N, K, y, ld_y};
  return hip_status(rmsn::launch_gemm(a, stream));
}

rmsn_status bigemm_bf16_tile(int64_t M, int64_t N, int64_t* tile_m, int64_t* tile_n) {
  if (M < 0 || N < 0) return RMSN_ERR_SHAPE;
  if (tile_m == nullptr || tile_n == nullptr) return RMSN_ERR_NULL;
  rmsn::gemm_tile(M, N, tile_m, tile_n);
  return RMSN_OK;
}

}  // extern "C"
