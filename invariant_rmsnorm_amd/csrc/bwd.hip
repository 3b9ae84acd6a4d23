// Backward launchers: the plain and residual-gradient rows kernels (the
// template is in bwd_kernel.hpp; the gated forms are in bwd_gated.hip, the
// fused add-norm forms in bwd_add.hip, fp16 activations in bwd_f16.hip) and
// the dgamma finish kernel.
//
// Finish: dgamma[j] = a fixed tree over 16 slices, each slice an ascending
// sum over a contiguous range of the chunk partials. The grouping depends on
// T (dgamma is a sum over the whole batch) but never on timing: the bits
// repeat run to run.
#include "bwd_kernel.hpp"

namespace rmsn {

// dgamma from the chunk partials (rows of Dp = part_stride(D) floats). A
// workgroup is two waves covering 32 columns (one 128-byte line of each
// partial row, so no line is fetched by two workgroups); in wave w, lane =
// 16*q + s, where q picks one of the wave's 4 float4 groups and s one of 16
// slices. Slice s sums its contiguous range of chunks in ascending order
// (its loads issued together), then the 16 slice sums meet in the fixed DPP
// butterfly over the 16 lanes that share q. chunks == 0 writes zeros (the
// empty sum).
constexpr int kFinishSlices = 16;
constexpr int kFinishQuads = 64 / kFinishSlices;  // float4 groups per wave
constexpr int kFinishWaves = 2;
constexpr int kFinishLoads = 16;                  // loads in flight per lane

__global__ __launch_bounds__(64 * kFinishWaves) void rmsnorm_bwd_finish_kernel(
    const float* __restrict__ part, int64_t chunks, int D, float* __restrict__ dgamma) {
  const int lane = threadIdx.x & 63;
  const int q = lane / kFinishSlices;
  const int s = lane % kFinishSlices;
  const int col4 = (blockIdx.x * kFinishWaves + wave_id()) * kFinishQuads + q;
  const int d4 = static_cast<int>(part_stride(D)) >> 2;
  const int64_t per = (chunks + kFinishSlices - 1) / kFinishSlices;
  const int64_t k0 = s * per;
  const int64_t k1 = k0 + per < chunks ? k0 + per : chunks;
  // One resource over all partials (at most 512 x 2048 or 256 x 32768
  // floats, 32 MiB);
  // lanes past D and chunks past the slice's range get an offset beyond it
  // and read zeros, so the loads need no branches.
  const bool ok = col4 < d4;
  const auto rp = f32_rsrc(part, 0, chunks * d4 * 4, 0x7FFFFFFF / 4);
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int64_t kb = k0; kb < k1; kb += kFinishLoads) {
    u32x4 t[kFinishLoads];
#pragma unroll
    for (int j = 0; j < kFinishLoads; ++j) {
      const bool in = ok && kb + j < k1;
      t[j] = buf_load16(rp, in ? static_cast<uint32_t>(((kb + j) * d4 + col4) * 16) : kOutOfRange);
    }
#pragma unroll
    for (int j = 0; j < kFinishLoads; ++j) {
      if (kb + j < k1) {
        acc.x = acc.x + __uint_as_float(t[j].x); acc.y = acc.y + __uint_as_float(t[j].y);
        acc.z = acc.z + __uint_as_float(t[j].z); acc.w = acc.w + __uint_as_float(t[j].w);
      }
    }
  }
  acc.x = row_sum<kFinishSlices>(acc.x);
  acc.y = row_sum<kFinishSlices>(acc.y);
  acc.z = row_sum<kFinishSlices>(acc.z);
  acc.w = row_sum<kFinishSlices>(acc.w);
  if (s == 0 && ok) {
    if (4 * col4 + 4 <= D) {
      reinterpret_cast<float4*>(dgamma)[col4] = acc;
    } else {
      // the columns of the last group that lie inside the row
      const float v[4] = {acc.x, acc.y, acc.z, acc.w};
      for (int e = 0; e < 4 && 4 * col4 + e < D; ++e) dgamma[4 * col4 + e] = v[e];
    }
  }
}

int launch_bwd_rows(const BwdArgs& a, void* stream) {
  if (a.T == 0 || a.chunks == 0) return 0;
  if (a.z != nullptr) return launch_bwd_rows_gated(a, stream);
  if (a.rin != nullptr) return launch_bwd_rows_add(a, stream);
  if (a.D % 8 != 0) return launch_bwd_rows_elem(a, stream);
  if (a.dt == kF16) return launch_bwd_rows_f16(a, stream);
  const RowGeom g = bwd_geom(a.D);
  const bwd_detail::RowsLaunch f =
      a.gres != nullptr ? bwd_detail::pick<kBwdGres>(g) : bwd_detail::pick<kBwdPlain>(g);
  if (f == nullptr) return static_cast<int>(hipErrorInvalidValue);
  return f(a, stream);
}

int launch_bwd_finish(const float* part, int64_t chunks, int D, float* dgamma, void* stream) {
  const int cols_per_block = 4 * kFinishQuads * kFinishWaves;
  const int grid = static_cast<int>((part_stride(D) + cols_per_block - 1) / cols_per_block);
  hipLaunchKernelGGL(rmsnorm_bwd_finish_kernel, dim3(grid), dim3(64 * kFinishWaves), 0,
                     static_cast<hipStream_t>(stream), part, chunks, D, dgamma);
  return static_cast<int>(hipGetLastError());
}

}  // namespace rmsn
