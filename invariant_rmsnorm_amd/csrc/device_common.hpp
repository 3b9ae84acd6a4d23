// Device helpers for the gfx950 RMSNorm kernels: bf16 widening and
// narrowing, 16-byte vector access, and the fixed within-row reduction tree.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "geometry.hpp"

namespace rmsn {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Unpack the 8 bf16 values of a 16-byte vector, in memory order.
__device__ __forceinline__ void unpack8(const uint4& q, float (&f)[8]) {
  f[0] = bf16_lo(q.x); f[1] = bf16_hi(q.x);
  f[2] = bf16_lo(q.y); f[3] = bf16_hi(q.y);
  f[4] = bf16_lo(q.z); f[5] = bf16_hi(q.z);
  f[6] = bf16_lo(q.w); f[7] = bf16_hi(q.w);
}

// fp32 pair -> packed bf16 pair with round-to-nearest-even (one
// v_cvt_pk_bf16_f32 on gfx950); the first value lands in the low half.
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f32x2 v = {a, b};
  const bf16x2 h = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  return uint4{pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7])};
}

__device__ __forceinline__ uint4 load16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void store16_stream(uint16_t* p, const uint4& v) {
  const u32x4 q = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(q, reinterpret_cast<u32x4*>(p));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum of v over the LPR consecutive lanes that share a row, returned to all
// of them with identical bits. The tree is a butterfly: at every stage a lane
// adds its partner's value to its own (lane i and its partner compute a+b
// and b+a, equal in IEEE arithmetic), pairing lanes at distance 1, 2, then
// mirrored halves of 8 and of 16 lanes (DPP), then 16 apart (ds_swizzle),
// then the two halves of the wave. Its shape depends on LPR only. All 64
// lanes must be active.
template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
  if constexpr (LPR >= 2) v = v + dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  if constexpr (LPR >= 4) v = v + dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  if constexpr (LPR >= 8) v = v + dpp<0x141>(v);   // row_half_mirror
  if constexpr (LPR >= 16) v = v + dpp<0x140>(v);  // row_mirror
  if constexpr (LPR >= 32)                          // lanes i and i^16
    v = v + __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
  if constexpr (LPR >= 64) {                        // the two 32-lane halves
    const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    v = lo + hi;
  }
  return v;
}

// Loads this lane's weights w_eff = gamma (+1.0f in fp32 when zero-centred)
// for its vectors c = v*LPR + l; columns past D read as zero.
template <int LPR, int VPL, bool MASKED>
__device__ __forceinline__ void load_weights(const float* __restrict__ gamma, int zc, int nv,
                                             int l, float (&w)[VPL][8]) {
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int c = v * LPR + l;
    if (!MASKED || c < nv) {
      const float4 a = *reinterpret_cast<const float4*>(gamma + 8 * c);
      const float4 b = *reinterpret_cast<const float4*>(gamma + 8 * c + 4);
      w[v][0] = a.x; w[v][1] = a.y; w[v][2] = a.z; w[v][3] = a.w;
      w[v][4] = b.x; w[v][5] = b.y; w[v][6] = b.z; w[v][7] = b.w;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) w[v][k] = 0.0f;
    }
    if (zc) {
#pragma unroll
      for (int k = 0; k < 8; ++k) w[v][k] = w[v][k] + 1.0f;
    }
  }
}

}  // namespace rmsn
