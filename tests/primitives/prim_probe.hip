// Test helper (not part of the library): runs the library's device
// primitives on arbitrary inputs so the tests can check them element by
// element: the fp32 -> bf16 pair conversion the kernels store with
// (rmsn::pack2, gfx950's v_cvt_pk_bf16_f32) and the gate functions of the
// gated norm (the forward's sigmoid_fast / gate_fast, the backward's gate and
// gate_and_grad). Every kernel is a bounds-checked grid-stride loop.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace {

// out[i] = bf16 bits of the fp32 value whose bits are first + i, i < n, two
// values per conversion (the low and the high half of one packed result).
__global__ void pack_all(uint32_t first, int64_t n, uint16_t* out) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x * 2;
  for (int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 2; i < n;
       i += stride) {
    const float a = __uint_as_float(first + static_cast<uint32_t>(i));
    const float b = __uint_as_float(first + static_cast<uint32_t>(i + 1));
    const uint32_t p = rmsn::pack2(a, b);
    out[i] = static_cast<uint16_t>(p & 0xFFFFu);
    if (i + 1 < n) out[i + 1] = static_cast<uint16_t>(p >> 16);
  }
}

// For each z: [sigmoid_fast, gate_fast<silu>, gate<sigmoid>, gate<silu>,
// d/dz sigmoid, d/dz silu] (the last two from gate_and_grad).
__global__ void gates(const float* z, int64_t n, float* out) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float v = z[i];
    float* o = out + 6 * i;
    o[0] = rmsn::sigmoid_fast(v);
    o[1] = rmsn::gate_fast<rmsn::kGateSilu>(v);
    o[2] = rmsn::gate<rmsn::kGateSigmoid>(v);
    o[3] = rmsn::gate<rmsn::kGateSilu>(v);
    float a, da;
    rmsn::gate_and_grad<rmsn::kGateSigmoid>(v, a, da);
    o[4] = da;
    rmsn::gate_and_grad<rmsn::kGateSilu>(v, a, da);
    o[5] = da;
  }
}

}  // namespace

extern "C" int prim_pack_all(uint32_t first, int64_t n, uint16_t* out, void* stream) {
  if (n <= 0 || out == nullptr || n > (int64_t{1} << 32)) return -1;
  hipLaunchKernelGGL(pack_all, dim3(4096), dim3(256), 0, static_cast<hipStream_t>(stream), first, n, out);
  return static_cast<int>(hipGetLastError());
}

extern "C" int prim_gates(const float* z, int64_t n, float* out, void* stream) {
  if (n <= 0 || z == nullptr || out == nullptr) return -1;
  hipLaunchKernelGGL(gates, dim3(2048), dim3(256), 0, static_cast<hipStream_t>(stream), z, n, out);
  return static_cast<int>(hipGetLastError());
}
