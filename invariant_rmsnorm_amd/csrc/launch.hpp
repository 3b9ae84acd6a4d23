// Host-side interface between the C-ABI entry points (api.cpp) and the
// kernel launchers (fwd.hip, bwd.hip). Plain types only: api.cpp does not
// include any HIP header. Arguments arrive already validated.
#pragma once

#include <stdint.h>

namespace rmsn {

struct FwdArgs {
  const uint16_t* x;
  int64_t ld_x;
  const uint16_t* z;  // gate, or nullptr
  int64_t ld_z;
  const float* gamma;
  int zc;
  float eps;
  int64_t T;
  int D;
  uint16_t* y;
  int64_t ld_y;
  uint16_t* res;  // residual copy, or nullptr
  int64_t ld_res;
  float* rstd;  // or nullptr
};

struct BwdArgs {
  const uint16_t* g;
  int64_t ld_g;
  const uint16_t* x;
  int64_t ld_x;
  const float* rstd;
  const float* gamma;
  int zc;
  int64_t T;
  int D;
  const uint16_t* gres;  // or nullptr
  int64_t ld_gres;
  uint16_t* dx;  // or nullptr
  int64_t ld_dx;
  float* part;  // [chunks][D] dgamma partials, or nullptr
  int64_t chunk_rows;
  int64_t chunks;
};

// Each returns 0 on success or the HIP error code of a refused launch.
int launch_fwd(const FwdArgs& a, void* stream);
int launch_bwd_rows(const BwdArgs& a, void* stream);
int launch_bwd_finish(const float* part, int64_t chunks, int D, float* dgamma, void* stream);

}  // namespace rmsn
