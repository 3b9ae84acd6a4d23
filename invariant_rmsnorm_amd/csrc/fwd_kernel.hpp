// Forward kernel template: plain, residual-copy and gated RMSNorm over the
// last axis of a [T, D] bf16 tensor, for gfx950. fwd.hip instantiates the
// ungated forms, fwd_gated.hip the gated ones (built apart, in parallel).
//
// What a row computes follows Megatron-LM PR "Fix the batch-invariant RMSNorm
// forward and its input gradient" (item 1: w_eff = fp32(gamma) + 1 when
// zero-centred), RL-Kernel PR "[DSv4][P1-5] rmsnorm_residual"
// ("Implementation": r = rsqrt(mean(x^2) + eps), y = (x * r) * gamma, mul and
// add rounded separately; "Summary": the residual output is a byte copy of x)
// and RL-Kernel PR "C1: zero-centred RMSNorm references and CUDA kernel" (the
// gated norm: out = norm * a(z), a = silu or sigmoid; one upstream does the
// weight multiply in fp32, the other casts to the input dtype first).
//
// Work split. A 256-thread workgroup is 4 waves; each wave processes U*RPW
// rows per step (RPW = 64/LPR rows side by side, U steps unrolled so each
// lane has ~128 bytes of loads in flight), and workgroups stride over the
// batch. Per row: 16-byte loads of x, the sum of squares of the lane's own
// elements in a fixed order, the fixed DPP butterfly over the row's lanes
// (row_sum), r, then y written with 16-byte non-temporal stores. None of
// these steps looks at T, the row index or the strides except to address
// memory, so each row's bits are the same in any batch.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include <algorithm>
#include <atomic>

#include "device_common.hpp"
#include "launch.hpp"

namespace rmsn {

// GATE: 0 = no gate; otherwise 1 + activation + 2 * cast, where cast selects
// the convention that rounds the normalised and the weighted value to the
// activations' storage type before the next multiply; kFwdAdd = the fused
// add-norm.
constexpr int fwd_gate_code(bool gated, int act, bool cast) { return gated ? 1 + act + 2 * cast : 0; }
constexpr int kFwdAdd = 5;

template <int LPR, int VPL, bool MASKED, int GATE, int DT>
__global__ __launch_bounds__(kBlock) void rmsnorm_fwd_kernel(FwdArgs a) {
  constexpr bool ADD = GATE == kFwdAdd;
  constexpr bool GATED = GATE != 0 && !ADD;
  constexpr int ACT = GATED ? (GATE - 1) & 1 : 0;
  constexpr bool CAST = GATED && (GATE - 1) >= 2;
  constexpr int RPW = rows_per_wave(LPR);
  constexpr int WPR = waves_per_row(LPR);
  constexpr int U = fwd_unroll(LPR, VPL);
  constexpr int ROWS_WAVE = U * RPW;
  constexpr int ROWS_BLOCK = rows_per_block(LPR, U);
  static_assert(WPR == 1 || (U == 1 && VPL >= kFwdMinVplMulti), "multi-wave rows: one row per step");
  // second input stream: the gate z, or the fused add's residual input
  constexpr bool TWO = GATED || ADD;
  constexpr int ZU = TWO ? U : 1;
  constexpr int ZV = TWO ? VPL : 1;

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  // the wave's row group and, within its row, the lane's index l (rows
  // spread over WPR waves: l = 64 * (wave % WPR) + lane)
  const int group = wave / WPR;
  const int slot = LPR >= 64 ? 0 : lane / LPR;
  const int l = LPR >= 64 ? (wave % WPR) * 64 + lane : lane % LPR;
  __shared__ double xch[2][kWaves];  // row-sum exchange of multi-wave rows
  int xstep = 0;
  const int nv = (a.D + 7) >> 3;  // groups of 8 elements (the last may be partial)
  const float Df = static_cast<float>(a.D);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * ROWS_BLOCK;

  constexpr bool ELEM = elem_dt(DT);
  // rows of any length: a partial last group is read as the row's last 16
  // bytes, except in rows shorter than one group (LPR == 1)
  constexpr bool TAIL = LPR > 1;
  float w[VPL][8];
  if constexpr (ELEM) load_weights_any<LPR, VPL>(a.gamma, a.wdt, a.zc, a.D, l, w);
  else load_weights<LPR, VPL, MASKED>(a.gamma, a.wdt, a.zc, nv, l, w);

  // Byte offset of this lane's group v (elements [8c, 8c + 8), c = v*LPR + l)
  // within its row group, per tensor. With 16-byte storage, groups past D
  // get an offset no resource reaches; in rows of any length the last
  // group's elements are checked one by one (`valid`: the row's elements from
  // the group's first on; `last`: only a lane's last group can be partial).
  auto voff = [&](int v, int64_t ld) -> uint32_t {
    const int c = v * LPR + l;
    if (!ELEM && MASKED && c >= nv) return kOutOfRange;
    return static_cast<uint32_t>(slot * ld * 2 + 16 * c);
  };
  auto valid = [&](int v) { return a.D - 8 * (v * LPR + l); };
  auto last = [](int v) { return v == VPL - 1; };
  // Rows first .. first+RPW-1 form row group u of the wave; `first` is
  // wave-uniform.
  auto group_first = [&](int64_t base, int u) { return base + group * ROWS_WAVE + u * RPW; };

  // The inputs' cache policy: the default keeps rows the backward reads
  // next in the Infinity Cache; inputs well past it take the streaming
  // hint (a wave-uniform choice).
  auto load_inputs = [&](auto policy, int64_t base, u32x4 (&xq)[U][VPL], u32x4 (&zq)[ZU][ZV]) {
    constexpr int P = decltype(policy)::value;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t first = group_first(base, u);
      const auto rx = rows_rsrc(a.x, first, a.T, RPW, a.ld_x, a.D);
#pragma unroll
      for (int v = 0; v < VPL; ++v) xq[u][v] = load_row8<DT, P, TAIL>(rx, voff(v, a.ld_x), valid(v), last(v));
      if constexpr (GATED) {
        const auto rz = rows_rsrc(a.z, first, a.T, RPW, a.ld_z, a.D);
#pragma unroll
        for (int v = 0; v < VPL; ++v) zq[u][v] = load_row8<DT, P, TAIL>(rz, voff(v, a.ld_z), valid(v), last(v));
      }
      if constexpr (ADD) {
        const auto rr = rows_rsrc(a.rin, first, a.T, RPW, a.ld_rin, a.D);
#pragma unroll
        for (int v = 0; v < VPL; ++v)
          zq[u][v] = load_row8<DT, P, TAIL>(rr, voff(v, a.ld_rin), valid(v), last(v));
      }
    }
  };
  auto load_step = [&](int64_t base, u32x4 (&xq)[U][VPL], u32x4 (&zq)[ZU][ZV]) {
    if (a.x_stream) load_inputs(std::integral_constant<int, kLoadStream>{}, base, xq, zq);
    else load_inputs(std::integral_constant<int, kLoadDefault>{}, base, xq, zq);
  };
  // The row's values as fp32: x, or for the fused add h = x + rin (one fp32
  // rounding).
  auto row_values = [&](const u32x4& xv, const u32x4& rv, float (&f)[8]) {
    unpack8<DT>(xv, f);
    if constexpr (ADD) {
      float rf[8];
      unpack8<DT>(rv, rf);
#pragma unroll
      for (int k = 0; k < 8; ++k) f[k] = f[k] + rf[k];
    }
  };

  auto process = [&](int64_t base, u32x4 (&xq)[U][VPL], u32x4 (&zq)[ZU][ZV]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t first = group_first(base, u);
      const int64_t row = first + slot;

      // sum of squares: this lane's elements in (vector, element) order, then
      // the row's fixed butterfly. Squares of bf16 values are exact in fp32;
      // those of the fused add's h are rounded to fp32 once. A partial last
      // group read as the row's last 16 bytes moves into place where it is
      // first used: moved at the top of the step, its shifts made the
      // compiler wait for all of the step's loads before the first vector.
      acc_t ssa = 0;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        if (v == VPL - 1) {
          place_row8<DT, TAIL>(xq[u][VPL - 1], valid(VPL - 1), true);
          if constexpr (ADD) place_row8<DT, TAIL>(zq[u][VPL - 1], valid(VPL - 1), true);
        }
        float f[8];
        row_values(xq[u][v], zq[ADD ? u : 0][ADD ? v : 0], f);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float sq = f[k] * f[k];
          ssa = acc_add(ssa, sq);
        }
      }
      const float ss = static_cast<float>(row_total<LPR>(ssa, xch, xstep));
      const float r = rstd_of(ss, Df, a.eps);
      if constexpr (GATED) place_row8<DT, TAIL>(zq[u][VPL - 1], valid(VPL - 1), true);
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        opaque(xq[u][v]);
        if constexpr (ADD) opaque(zq[u][v]);
      }

      if (a.rstd != nullptr && l == 0 && row < a.T) a.rstd[row] = r;
      // rows past T: the resources below are empty and drop the stores
      const auto ry = rows_rsrc(a.y, first, a.T, RPW, a.ld_y, a.D);
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        float f[8], o[8];
        row_values(xq[u][v], zq[ADD ? u : 0][ADD ? v : 0], f);
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = f[k] * r;
        if constexpr (CAST) round8<DT>(o);
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = o[k] * w[v][k];
        if constexpr (GATED) {
          if constexpr (CAST) round8<DT>(o);
          float zf[8];
          unpack8<DT>(zq[u][v], zf);
#pragma unroll
          for (int k = 0; k < 8; ++k) o[k] = o[k] * gate_fast<ACT>(zf[k]);
        }
        store_row8<DT>(pack8<DT>(o), ry, voff(v, a.ld_y), valid(v), last(v));
      }
      if (a.res != nullptr) {
        // residual output: a byte copy of x, or for the fused add bf16(h)
        const auto rr = rows_rsrc(a.res, first, a.T, RPW, a.ld_res, a.D);
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          if constexpr (ADD) {
            float f[8];
            row_values(xq[u][v], zq[u][v], f);
            store_row8<DT>(pack8<DT>(f), rr, voff(v, a.ld_res), valid(v), last(v));
          } else {
            store_row8<DT>(xq[u][v], rr, voff(v, a.ld_res), valid(v), last(v));
          }
        }
      }
    }
  };

  for (int64_t base = static_cast<int64_t>(blockIdx.x) * ROWS_BLOCK; base < a.T; base += stride) {
    u32x4 xv[U][VPL];
    u32x4 zv[ZU][ZV];
    load_step(base, xv, zv);
    process(base, xv, zv);
  }
}

namespace fwd_detail {

inline int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Workgroups per launch, as a multiple of what fits on the device at once
// (1: a persistent grid). Every workgroup loads the row's weights before its
// first step, so the multiple shrinks as the weights grow. Measured on the
// plain forward with the cache flushed before each launch (us, x of 256 MiB;
// multiples 1 / 2 / 4 / 8 / 16):
//   D = 128    101.8 101.0  98.3  94.8  93.1
//   D = 4096   104.4 103.8 100.3  98.2  98.7  (T = 262144: 826 810 800 781 771)
//   D = 5120   106.5 110.5 103.8 102.1 100.3
//   D = 8192   114.6 110.4 110.2 118.7 119.6
//   D = 16384  109.9 106.2 105.7 111.3 111.5
//   D = 32768  114.1 108.7 109.1 111.0 111.2
// Re-measured on the present kernel, same box, x of 256 MiB, multiples 1 /
// 2 / 4: D = 8192 103.2 101.7 98.5, 12288 105.2 103.1 98.9, 16384 103.0
// 101.0 98.1, 20480 106.8 108.7 102.0, 24576 103.8 103.2 103.7, 28672 106.6
// 105.8 111.2, 32768 113.7 107.4 109.0; 4 against 2 at other batch sizes:
// D = 8192 T = 65536 394.9 -> 388.5, 10240 T = 13107 101.9 -> 97.0, 12288
// T = 9000 85.9 -> 81.4, 20480 T = 13107 208.3 -> 206.6, smaller batches
// within 1 us. Hence 4 up to 2560 groups per row (D = 20480) and 2 beyond.
constexpr int64_t fwd_grid_scale(int lpr, int vpl) {
  return lpr * vpl < 1024 ? 16 : lpr * vpl <= 2560 ? 4 : 2;
}

template <int LPR, int VPL, bool MASKED, int GATE, int DT>
int launch_inst(const FwdArgs& a, void* stream) {
  constexpr int ROWS_BLOCK = rows_per_block(LPR, fwd_unroll(LPR, VPL));
  auto kern = rmsnorm_fwd_kernel<LPR, VPL, MASKED, GATE, DT>;
  static const int per_cu = [&] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, kern, kBlock, 0) != hipSuccess || b < 1)
      b = 1;
    return b;
  }();
  // Grid: at most fwd_grid_scale times as many workgroups as fit on the
  // device at once (the hardware starts the rest as earlier ones finish, so
  // the last rows are shared by whichever compute units are free instead of
  // by a fixed set), and every workgroup given the same number of steps.
  const int64_t blocks = (a.T + ROWS_BLOCK - 1) / ROWS_BLOCK;
  const int64_t cap = static_cast<int64_t>(cu_count()) * per_cu * fwd_grid_scale(LPR, VPL);
  const int64_t steps = (blocks + cap - 1) / cap;
  const int grid = static_cast<int>(std::max<int64_t>(1, (blocks + steps - 1) / steps));
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kBlock), 0, static_cast<hipStream_t>(stream), a);
  return static_cast<int>(hipGetLastError());
}

using FwdLaunch = int (*)(const FwdArgs&, void*);

template <int GATE, int DT, int VPL = 1>
FwdLaunch pick_wide(int vpl, bool masked) {
  if constexpr (VPL > kMaxVpl) {
    return nullptr;
  } else {
    if (vpl == VPL)
      return masked ? &launch_inst<64, VPL, true, GATE, DT> : &launch_inst<64, VPL, false, GATE, DT>;
    return pick_wide<GATE, DT, VPL + 1>(vpl, masked);
  }
}

// Rows over several waves (D > 4096): 5 to 16 vectors per lane.
template <int GATE, int DT, int LPR, int VPL = kFwdMinVplMulti>
FwdLaunch pick_multi(int vpl, bool masked) {
  if constexpr (VPL > kMaxVpl) {
    return nullptr;
  } else {
    if (vpl == VPL)
      return masked ? &launch_inst<LPR, VPL, true, GATE, DT> : &launch_inst<LPR, VPL, false, GATE, DT>;
    return pick_multi<GATE, DT, LPR, VPL + 1>(vpl, masked);
  }
}

template <int GATE, int DT = kBf16>
FwdLaunch pick(const RowGeom& g) {
  switch (g.lpr) {
    case 256: return pick_multi<GATE, DT, 256>(g.vpl, g.masked);
    case 128: return pick_multi<GATE, DT, 128>(g.vpl, g.masked);
    case 64: return pick_wide<GATE, DT>(g.vpl, g.masked);
    case 32: return g.masked ? &launch_inst<32, 1, true, GATE, DT> : &launch_inst<32, 1, false, GATE, DT>;
    case 16: return g.masked ? &launch_inst<16, 1, true, GATE, DT> : &launch_inst<16, 1, false, GATE, DT>;
    case 8: return g.masked ? &launch_inst<8, 1, true, GATE, DT> : &launch_inst<8, 1, false, GATE, DT>;
    case 4: return g.masked ? &launch_inst<4, 1, true, GATE, DT> : &launch_inst<4, 1, false, GATE, DT>;
    case 2: return &launch_inst<2, 1, false, GATE, DT>;
    case 1: return &launch_inst<1, 1, false, GATE, DT>;
    default: return nullptr;
  }
}

}  // namespace fwd_detail
}  // namespace rmsn
