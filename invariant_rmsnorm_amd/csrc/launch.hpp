// Host-side interface between the C-ABI entry points (api.cpp) and the
// kernel launchers (fwd.hip, fwd_gated.hip, bwd.hip, bwd_gated.hip). Plain
// types only: api.cpp does not include any HIP header. Arguments arrive
// already validated.
#pragma once

#include <stdint.h>

namespace rmsn {

struct FwdArgs {
  const uint16_t* x;
  int64_t ld_x;
  const uint16_t* z;  // gate input, or nullptr (no gate)
  int64_t ld_z;
  int act;   // gate activation: 0 silu, 1 sigmoid
  int cast;  // gated rounding convention: 0 weight multiply in fp32, 1 casts
  const void* gamma;  // weights of storage type wdt
  int wdt;            // kBf16, kF16 or kF32
  int dt;             // activation storage type: kBf16 or kF16
  int zc;
  float eps;
  int64_t T;
  int D;
  uint16_t* y;
  int64_t ld_y;
  uint16_t* res;  // residual copy (bf16(x + rin) when rin is set), or nullptr
  int64_t ld_res;
  float* rstd;  // or nullptr
  const uint16_t* rin;  // fused add: residual input, normalise x + rin; or nullptr
  int64_t ld_rin;
  int x_stream;  // read x (z, rin) with the non-temporal hint (set by the caller)
};

struct BwdArgs {
  const uint16_t* g;
  int64_t ld_g;
  const uint16_t* x;
  int64_t ld_x;
  const float* rstd;
  const void* gamma;  // weights of storage type wdt
  int wdt;            // kBf16, kF16 or kF32
  int dt;             // activation storage type: kBf16 or kF16
  int zc;
  int64_t T;
  int D;
  const uint16_t* gres;  // or nullptr
  int64_t ld_gres;
  uint16_t* dx;  // or nullptr
  int64_t ld_dx;
  float* part;  // [chunks][D] dgamma partials, or nullptr
  int64_t chunks;
  int64_t group_blocks;  // row blocks per group of the chunk traversal
  // gated backward only (z == nullptr otherwise)
  const uint16_t* z;
  int64_t ld_z;
  int act;       // 0 silu, 1 sigmoid
  uint16_t* dz;  // or nullptr
  int64_t ld_dz;
  int x_stream;  // read x with the non-temporal hint (set by the launcher)
  const uint16_t* rin;  // fused add: residual input (h = x + rin); or nullptr
  int64_t ld_rin;
};

struct GemmArgs {
  const uint16_t* x;  // bf16 [M, K]
  int64_t ld_x;
  const uint16_t* w;  // bf16 [N, K]
  int64_t ld_w;
  int64_t M, N, K;
  uint16_t* y;  // bf16 [M, N]
  int64_t ld_y;
};

// Each returns 0 on success or the HIP error code of a refused launch.
int launch_fwd(const FwdArgs& a, void* stream);
int launch_fwd_gated(const FwdArgs& a, void* stream);  // a.z != nullptr
int launch_fwd_add(const FwdArgs& a, void* stream);    // a.rin != nullptr
int launch_fwd_f16(const FwdArgs& a, void* stream);
int launch_fwd_elem(const FwdArgs& a, void* stream);   // D % 8 != 0 (plain, residual copy)
int launch_fwd_gated_elem(const FwdArgs& a, void* stream);  // D % 8 != 0, gated
int launch_fwd_add_elem(const FwdArgs& a, void* stream);    // D % 8 != 0, fused add
int launch_fwd_gated_f16(const FwdArgs& a, void* stream);       // fp16, gated
int launch_fwd_gated_elem_f16(const FwdArgs& a, void* stream);  // fp16, gated, D % 8 != 0
int launch_fwd_add_f16(const FwdArgs& a, void* stream);         // fp16, fused add, any D
int launch_bwd_rows(const BwdArgs& a, void* stream);
int launch_bwd_rows_gated(const BwdArgs& a, void* stream);  // a.z != nullptr
int launch_bwd_rows_gated_elem(const BwdArgs& a, void* stream);  // a.z != nullptr, D % 8 != 0
int launch_bwd_rows_add(const BwdArgs& a, void* stream);    // a.rin != nullptr
int launch_bwd_rows_f16(const BwdArgs& a, void* stream);
int launch_bwd_rows_elem(const BwdArgs& a, void* stream);      // D % 8 != 0 (plain, gres)
int launch_bwd_rows_elem_f16(const BwdArgs& a, void* stream);  // the same, fp16 activations
int launch_bwd_rows_add_elem(const BwdArgs& a, void* stream);    // D % 8 != 0, fused add
int launch_bwd_rows_gated_f16(const BwdArgs& a, void* stream);       // fp16, gated
int launch_bwd_rows_gated_elem_f16(const BwdArgs& a, void* stream);  // fp16, gated, D % 8 != 0
int launch_bwd_rows_add_f16(const BwdArgs& a, void* stream);         // fp16, fused add, any D
int launch_bwd_finish(const float* part, int64_t chunks, int D, float* dgamma, void* stream);
int launch_gemm(const GemmArgs& a, void* stream);
// The output tile launch_gemm uses for an M x N product (host only).
void gemm_tile(int64_t M, int64_t N, int64_t* bm, int64_t* bn);

}  // namespace rmsn
