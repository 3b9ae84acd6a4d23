// Backward kernels for gfx950: the input gradient dx and the deterministic
// weight gradient dgamma.
//
// Formulas: Megatron-LM PR "Fix the batch-invariant RMSNorm forward and its
// input gradient", item 2 — with dr/dx_k = -r^3 x_k / D,
//     dx_k = g_k w_k r - (r^3 x_k / D) * sum_i g_i x_i w_i,
// the weight entering once in each term; RL-Kernel PR "[DSv4][P1-5]
// rmsnorm_residual", review comment — dx also receives the residual copy's
// gradient, and dgamma_j = sum over tokens of dy * x * r. The rstd used is
// the one the forward saved (RL-Kernel PR "C1: zero-centred RMSNorm
// references and CUDA kernel", parameter-VJP paragraph). No atomics, split-K
// or stream-K ("Implementation" of the rmsnorm_residual PR).
//
// Kernel 1 (rows): workgroup k owns the fixed chunk of rows
// [k*C, min(T,(k+1)*C)). Its waves walk the chunk in steps; per row a wave
// forms gw = g*w, the lane partial of s = sum gw*x, the fixed butterfly
// (same shape as the forward's), c = ((r*r)*r)*s/D and dx = gw*r - x*c
// (+ gres), stored with 16-byte non-temporal stores. For dgamma each lane
// keeps fp32 accumulators for the columns it owns, adding (g*x)*r row after
// row in chunk order. At the end of the chunk the row slots of a wave are
// added by a butterfly, the 4 waves as ((w0 + w2) + (w1 + w3)) through LDS,
// and the chunk's partial row is written to workspace[k][:].
// Kernel 2 (finish): dgamma[j] = a fixed tree over 32 slices, each slice an
// ascending sum over k of the partials. The grouping depends on T (dgamma is
// a sum over the whole batch) but never on timing: the bits repeat run to run.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace rmsn {

template <int LPR, int VPL, bool MASKED>
__global__ __launch_bounds__(kBlock) void rmsnorm_bwd_rows_kernel(BwdArgs a) {
  constexpr int RPW = 64 / LPR;
  constexpr int U = bwd_unroll(LPR, VPL);
  constexpr int ROWS_WAVE = U * RPW;
  constexpr int ROWS_BLOCK = kWaves * ROWS_WAVE;
  extern __shared__ float lds[];  // [2][D] when dgamma partials are wanted

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int slot = lane / LPR;
  const int l = lane % LPR;
  const int nv = a.D >> 3;
  const float Df = static_cast<float>(a.D);
  const bool want_dx = a.dx != nullptr;
  const bool want_part = a.part != nullptr;

  float w[VPL][8];
  load_weights<LPR, VPL, MASKED>(a.gamma, a.zc, nv, l, w);

  float acc[VPL][8];
#pragma unroll
  for (int v = 0; v < VPL; ++v)
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[v][k] = 0.0f;

  const int64_t begin = static_cast<int64_t>(blockIdx.x) * a.chunk_rows;
  const int64_t end = begin + a.chunk_rows < a.T ? begin + a.chunk_rows : a.T;

  for (int64_t step = begin; step < end; step += ROWS_BLOCK) {
    const int64_t row0 = step + wave * ROWS_WAVE + slot;
    uint4 gv[U][VPL], xv[U][VPL];
    float r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = row0 + u * RPW;
      const bool valid = row < end;
      r[u] = valid ? a.rstd[row] : 0.0f;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const int c = v * LPR + l;
        const bool ok = valid && (!MASKED || c < nv);
        gv[u][v] = ok ? load16(a.g + row * a.ld_g + 8 * c) : uint4{0, 0, 0, 0};
        xv[u][v] = ok ? load16(a.x + row * a.ld_x + 8 * c) : uint4{0, 0, 0, 0};
      }
    }

#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = row0 + u * RPW;
      const bool valid = row < end;

      if (want_dx) {
        // s = sum_i (g_i * w_i) * x_i: lane partial in (vector, element)
        // order, then the row's fixed butterfly.
        float s = 0.0f;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          float gf[8], xf[8];
          unpack8(gv[u][v], gf);
          unpack8(xv[u][v], xf);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float gw = gf[k] * w[v][k];
            s = __builtin_fmaf(gw, xf[k], s);
          }
        }
        s = row_sum<LPR>(s);
        const float rr = r[u] * r[u];
        const float r3 = rr * r[u];
        const float r3s = r3 * s;
        const float c = r3s / Df;

        if (valid) {
#pragma unroll
          for (int v = 0; v < VPL; ++v) {
            const int cv = v * LPR + l;
            if (MASKED && cv >= nv) continue;
            float gf[8], xf[8], o[8];
            unpack8(gv[u][v], gf);
            unpack8(xv[u][v], xf);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const float gw = gf[k] * w[v][k];
              const float t1 = gw * r[u];
              const float t2 = xf[k] * c;
              o[k] = t1 - t2;
            }
            if (a.gres != nullptr) {
              float rf[8];
              unpack8(load16(a.gres + row * a.ld_gres + 8 * cv), rf);
#pragma unroll
              for (int k = 0; k < 8; ++k) o[k] = o[k] + rf[k];
            }
            store16_stream(a.dx + row * a.ld_dx + 8 * cv, pack8(o));
          }
        }
      }

      if (want_part) {
        // (g*x) is exact in fp32 for bf16 inputs; one rounding per row.
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          float gf[8], xf[8];
          unpack8(gv[u][v], gf);
          unpack8(xv[u][v], xf);
#pragma unroll
          for (int k = 0; k < 8; ++k) acc[v][k] = __builtin_fmaf(gf[k] * xf[k], r[u], acc[v][k]);
        }
      }
    }
  }

  if (!want_part) return;

  // Row slots of one wave hold different rows of the same columns: add them
  // with a butterfly over the slot bits (every slot ends with equal bits).
#pragma unroll
  for (int m = LPR; m < 64; m <<= 1)
#pragma unroll
    for (int v = 0; v < VPL; ++v)
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[v][k] = acc[v][k] + __shfl_xor(acc[v][k], m);

  // Waves: ((w0 + w2) + (w1 + w3)) through two LDS rows of D floats.
  const bool writer = slot == 0;
  auto lds_row = [&](int b) { return lds + b * a.D; };
  if (wave >= 2 && writer) {
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int c = v * LPR + l;
      if (MASKED && c >= nv) continue;
      float* d = lds_row(wave - 2) + 8 * c;
      *reinterpret_cast<float4*>(d) = make_float4(acc[v][0], acc[v][1], acc[v][2], acc[v][3]);
      *reinterpret_cast<float4*>(d + 4) = make_float4(acc[v][4], acc[v][5], acc[v][6], acc[v][7]);
    }
  }
  __syncthreads();
  if (wave < 2 && writer) {
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int c = v * LPR + l;
      if (MASKED && c >= nv) continue;
      float* d = lds_row(wave) + 8 * c;
      const float4 p0 = *reinterpret_cast<const float4*>(d);
      const float4 p1 = *reinterpret_cast<const float4*>(d + 4);
      acc[v][0] = acc[v][0] + p0.x; acc[v][1] = acc[v][1] + p0.y;
      acc[v][2] = acc[v][2] + p0.z; acc[v][3] = acc[v][3] + p0.w;
      acc[v][4] = acc[v][4] + p1.x; acc[v][5] = acc[v][5] + p1.y;
      acc[v][6] = acc[v][6] + p1.z; acc[v][7] = acc[v][7] + p1.w;
      if (wave == 1) {  // the same wave read this row just above
        *reinterpret_cast<float4*>(d) = make_float4(acc[v][0], acc[v][1], acc[v][2], acc[v][3]);
        *reinterpret_cast<float4*>(d + 4) = make_float4(acc[v][4], acc[v][5], acc[v][6], acc[v][7]);
      }
    }
  }
  __syncthreads();
  if (wave == 0 && writer) {
    float* out = a.part + static_cast<int64_t>(blockIdx.x) * a.D;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int c = v * LPR + l;
      if (MASKED && c >= nv) continue;
      const float* d = lds_row(1) + 8 * c;
      const float4 p0 = *reinterpret_cast<const float4*>(d);
      const float4 p1 = *reinterpret_cast<const float4*>(d + 4);
      const float4 o0 = make_float4(acc[v][0] + p0.x, acc[v][1] + p0.y, acc[v][2] + p0.z, acc[v][3] + p0.w);
      const float4 o1 = make_float4(acc[v][4] + p1.x, acc[v][5] + p1.y, acc[v][6] + p1.z, acc[v][7] + p1.w);
      *reinterpret_cast<float4*>(out + 8 * c) = o0;
      *reinterpret_cast<float4*>(out + 8 * c + 4) = o1;
    }
  }
}

// dgamma from the chunk partials. A workgroup covers 32 columns (8 float4
// groups) with 32 k-slices; slice s sums k = s, s+32, s+64, ... in ascending
// order, then the 32 slice sums meet in a fixed halving tree in LDS.
// chunks == 0 writes zeros (the empty sum).
constexpr int kFinishSlices = 32;
constexpr int kFinishQuads = kBlock / kFinishSlices;  // float4 groups per block

__global__ __launch_bounds__(kBlock) void rmsnorm_bwd_finish_kernel(const float* __restrict__ part,
                                                                    int64_t chunks, int D,
                                                                    float* __restrict__ dgamma) {
  __shared__ float4 red[kFinishSlices][kFinishQuads];
  const int q = threadIdx.x % kFinishQuads;
  const int s = threadIdx.x / kFinishQuads;
  const int col4 = blockIdx.x * kFinishQuads + q;
  const int d4 = D >> 2;
  const bool ok = col4 < d4;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (ok) {
    const float4* p = reinterpret_cast<const float4*>(part) + col4;
    for (int64_t k = s; k < chunks; k += kFinishSlices) {
      const float4 t = p[k * d4];
      acc.x = acc.x + t.x; acc.y = acc.y + t.y; acc.z = acc.z + t.z; acc.w = acc.w + t.w;
    }
  }
  red[s][q] = acc;
  __syncthreads();
#pragma unroll
  for (int h = kFinishSlices / 2; h >= 1; h >>= 1) {
    if (s < h) {
      const float4 o = red[s + h][q];
      float4 m = red[s][q];
      m.x = m.x + o.x; m.y = m.y + o.y; m.z = m.z + o.z; m.w = m.w + o.w;
      red[s][q] = m;
    }
    __syncthreads();
  }
  if (s == 0 && ok) reinterpret_cast<float4*>(dgamma)[col4] = red[0][q];
}

namespace {

template <int LPR, int VPL, bool MASKED>
int launch_rows_inst(const BwdArgs& a, void* stream) {
  const size_t lds = a.part != nullptr ? 2 * sizeof(float) * static_cast<size_t>(a.D) : 0;
  hipLaunchKernelGGL((rmsnorm_bwd_rows_kernel<LPR, VPL, MASKED>), dim3(static_cast<unsigned>(a.chunks)),
                     dim3(kBlock), lds, static_cast<hipStream_t>(stream), a);
  return static_cast<int>(hipGetLastError());
}

using RowsLaunch = int (*)(const BwdArgs&, void*);

template <int VPL = 1>
RowsLaunch pick_wide(int vpl, bool masked) {
  if constexpr (VPL > kMaxVpl) {
    return nullptr;
  } else {
    if (vpl == VPL) return masked ? &launch_rows_inst<64, VPL, true> : &launch_rows_inst<64, VPL, false>;
    return pick_wide<VPL + 1>(vpl, masked);
  }
}

RowsLaunch pick(const RowGeom& g) {
  switch (g.lpr) {
    case 64: return pick_wide(g.vpl, g.masked);
    case 32: return g.masked ? &launch_rows_inst<32, 1, true> : &launch_rows_inst<32, 1, false>;
    case 16: return g.masked ? &launch_rows_inst<16, 1, true> : &launch_rows_inst<16, 1, false>;
    case 8: return g.masked ? &launch_rows_inst<8, 1, true> : &launch_rows_inst<8, 1, false>;
    case 4: return g.masked ? &launch_rows_inst<4, 1, true> : &launch_rows_inst<4, 1, false>;
    case 2: return &launch_rows_inst<2, 1, false>;
    case 1: return &launch_rows_inst<1, 1, false>;
    default: return nullptr;
  }
}

}  // namespace

int launch_bwd_rows(const BwdArgs& a, void* stream) {
  if (a.T == 0 || a.chunks == 0) return 0;
  const RowsLaunch f = pick(row_geom(a.D));
  if (f == nullptr) return static_cast<int>(hipErrorInvalidValue);
  return f(a, stream);
}

int launch_bwd_finish(const float* part, int64_t chunks, int D, float* dgamma, void* stream) {
  const int cols_per_block = 4 * kFinishQuads;
  const int grid = (D + cols_per_block - 1) / cols_per_block;
  hipLaunchKernelGGL(rmsnorm_bwd_finish_kernel, dim3(grid), dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), part, chunks, D, dgamma);
  return static_cast<int>(hipGetLastError());
}

}  // namespace rmsn
