// Batch-invariant BF16 GEMM Y = X @ W.T on gfx950 matrix cores.
//
// TransformerEngine issue "Expose Batch Invariant Kernels", point 3: the
// library GEMM was not batch-invariant because the algorithm (and with it
// the reduction order) was chosen from the whole problem shape; a GEMM whose
// output tiles accumulate over K in a fixed BLOCK_K loop, with the tile grid
// derived from tile coordinates only and no split-K, is invariant. Here:
//  - one tile geometry for every shape: 256 x 128 outputs per workgroup,
//    4 waves of 128 x 64 each, MFMA 32x32x16 bf16 with fp32 accumulation;
//  - K in steps of 32 (two MFMA k-steps), always ascending, each step
//    staged through LDS (double-buffered: the next step's global loads are
//    in flight while this one multiplies);
//  - rows of X past M and rows of W past N read as zero (buffer resources),
//    and outputs past M or N are not stored, so a row of Y is computed the
//    same way whatever M is.
// X [M, K] and W [N, K] are row-major with K contiguous: MFMA lane l takes
// 8 consecutive k of row l % 32 at k-offset 8 * (l / 32) for both operands,
// and holds output rows 8 * (r / 4) + 4 * (l / 32) + r % 4 (r = 0..15) of
// column l % 32.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace rmsn {

namespace {

constexpr int kBM = 256, kBN = 128, kBK = 32;
constexpr int kLdsRow = kBK + 8;  // bf16 per LDS row: 64 B of data + 16 B of padding

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void bigemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kBN * kLdsRow];

  const int64_t tiles_n = (a.N + kBN - 1) / kBN;
  const int64_t m0 = (static_cast<int64_t>(blockIdx.x) / tiles_n) * kBM;
  const int64_t n0 = (static_cast<int64_t>(blockIdx.x) % tiles_n) * kBN;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = wave_id();
  const int wm = wave >> 1, wn = wave & 1;

  // The tile's rows of X and of W (rows past M or N are outside the
  // resources and read as zero).
  const auto rx = rows_rsrc(a.x, m0, a.M, kBM, a.ld_x, static_cast<int>(a.K));
  const auto rw = rows_rsrc(a.w, n0, a.N, kBN, a.ld_w, static_cast<int>(a.K));

  // Global -> registers -> LDS: 16-byte chunk q of a stage is row q / 4,
  // columns 8 * (q % 4) .. +8 of the 32 k of the stage.
  u32x4 ga[4], gb[2];
  auto load_global = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = t + 256 * i;
      ga[i] = buf_load16(rx, static_cast<uint32_t>(((q >> 2) * a.ld_x + k0 + 8 * (q & 3)) * 2));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = t + 256 * i;
      gb[i] = buf_load16(rw, static_cast<uint32_t>(((q >> 2) * a.ld_w + k0 + 8 * (q & 3)) * 2));
    }
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = t + 256 * i;
      *reinterpret_cast<u32x4*>(&As[buf][(q >> 2) * kLdsRow + 8 * (q & 3)]) = ga[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = t + 256 * i;
      *reinterpret_cast<u32x4*>(&Bs[buf][(q >> 2) * kLdsRow + 8 * (q & 3)]) = gb[i];
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  auto compute = [&](int buf) {
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const int kk = 16 * s + 8 * (lane >> 5);
      bf16x8 fa[4], fb[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(
            &As[buf][(wm * 128 + 32 * i + (lane & 31)) * kLdsRow + kk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[j] = *reinterpret_cast<const bf16x8*>(
            &Bs[buf][(wn * 64 + 32 * j + (lane & 31)) * kLdsRow + kk]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  };

  const int64_t nk = a.K / kBK;
  load_global(0);
  store_lds(0);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = static_cast<int>(kt & 1);
    if (kt + 1 < nk) load_global((kt + 1) * kBK);
    compute(cur);
    // the other buffer was last read in the previous step, before its barrier
    if (kt + 1 < nk) store_lds(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: each fp32 sum rounded once to bf16; lanes 0..31 store 32
  // consecutive columns of one row, lanes 32..63 the same columns 4 rows on.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 64 + 32 * j + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 128 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < a.M && col < a.N)
          a.y[row * a.ld_y + col] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[i][j][r]));
      }
    }
}

}  // namespace

int launch_gemm(const GemmArgs& a, void* stream) {
  if (a.M == 0 || a.N == 0) return 0;
  const int64_t tiles = ((a.M + kBM - 1) / kBM) * ((a.N + kBN - 1) / kBN);
  hipLaunchKernelGGL(bigemm_kernel, dim3(static_cast<unsigned>(tiles)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return static_cast<int>(hipGetLastError());
}

}  // namespace rmsn
