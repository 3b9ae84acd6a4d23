// Backward rows kernel template for gfx950: the input gradient dx and the
// per-chunk dgamma partials; for the gated norm also the gate gradient dz.
// bwd.hip instantiates the plain and residual-gradient forms (and holds the
// finish kernel), bwd_gated.hip the gated forms (built apart, in parallel).
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
// Gated norm (out = n * w * a(z), n = x * r; the pages give its forward
// only, the backward here is the chain rule): the gradient reaching the
// normalised value is gn = g * a(z), which then takes the place of g in the
// formulas above (dx and dgamma); the gate's own gradient is
// dz = (g * (n * w)) * a'(z).
//
// Work split: workgroup k owns dgamma chunk k, a fixed set of row blocks
// spread over the batch (bwd_plan in geometry.hpp). Its waves walk the
// chunk's blocks in steps; per row a wave forms gw = g*w, the lane
// partial of s = sum gw*x, the fixed butterfly (same shape as the forward's),
// c = ((r*r)*r)*s/D and dx = gw*r - x*c (+ gres), stored with 16-byte
// non-temporal stores. For dgamma each lane keeps fp32 accumulators for the
// columns it owns, adding (g*x)*r row after row in chunk order. At the end of
// the chunk the row slots of a wave are added by a butterfly, the 4 waves as
// ((w0 + w2) + (w1 + w3)) through LDS, and the chunk's partial row is written
// to workspace[k][:].
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace rmsn {

// What the rows kernel computes besides plain dx / dgamma. The fused add
// modes take h = x + rin (fp32) in place of x and write the one gradient dh
// of both inputs; kBwdAddGres adds the gradient arriving at the updated
// residual (in the gres slot).
enum : int {
  kBwdPlain = 0, kBwdGres = 1, kBwdGatedSilu = 2, kBwdGatedSigmoid = 3,
  kBwdAdd = 4, kBwdAddGres = 5
};

// Register plan by geometry (chosen by measurement at D=4096; results do not
// depend on it). The kernel runs one 4-wave workgroup per compute unit, so
// each wave may use the whole register file. Up to 12 vectors per lane the
// weights stay in registers and the values unpacked in the first pass are
// reused by the second. Beyond that the registers would spill, so the
// weights move to LDS and the second pass unpacks the raw vectors again.
// The gated form holds a third input row (z), so it goes lean from 11.
// Rows of any length hold their groups as 16-byte vectors too and take the
// same plan.
constexpr bool bwd_lean(int vpl, bool three_inputs) { return vpl >= (three_inputs ? 11 : 13); }
// Load the next step while computing this one (two register sets that swap
// roles) where a wave would otherwise leave the memory pipe idle while it
// computes, and the loaded step fits the register file twice without
// scratch, checked with the compiler's resource report for every instance
// (with the whole register file, VPL <= 9 and input streams x VPL <= 24 for
// 16-byte rows over 4 waves: plain 9, three streams 8, four 6; 21 for bf16
// rows of any length over 4 waves without the gate; 18 for one-wave rows
// and the other rows of any length, whose lane offsets and tail shifts take
// more registers; at two waves per SIMD, streams x VPL <= 8). Residual
// gradient, same box, us per 256 MiB of x: D = 12290 (any length, 7
// vectors) 233.3 -> 211.1 cache evicted with the cap raised from 18 to 21;
// D = 16384 (8 vectors) 220.3 -> 200.3 after the forward, from 21 to 24.
//  - rows over 4 waves: held together by the exchange barrier, the waves
//    load and compute in lock step;
//  - one-wave rows from 5 vectors per lane on, where a wave is alone on its
//    SIMD. Measured against no prefetch (us per 256 MiB of x, cache evicted
//    / warm): D = 2050 158.2 / 169.3 -> 152.6 / 144.4, 4096 148.3 / 138.2 ->
//    146.7 / 140.8, 3072 144.5 / 138.0 -> 146.0 / 135.7. With two waves per
//    SIMD it cost 1-2% (D = 1000, 2048), so narrower rows go without.
// At two waves per SIMD only the gated rows over 4 waves take a third
// stream at 3 vectors: their gate arithmetic is long enough that the other
// workgroup does not hide it (D = 4100 447.1 -> 329.9 us, 4104 446.5 ->
// 316.1, same box, cache evicted); the residual gradient and the fused add
// measured slower that way (D = 8192 198.4 -> 206.2, fused add 4104 249.2
// -> 257.9), and the gated rows at 4 vectors no faster.
constexpr bool bwd_prefetch(int lpr, int vpl, int mode, int dt) {
  const int streams = 2 + (mode == kBwdPlain ? 0 : 1) + (mode == kBwdAddGres ? 1 : 0);
  const bool gated = mode == kBwdGatedSilu || mode == kBwdGatedSigmoid;
  const int cap = lpr <= 64 ? 18 : !elem_dt(dt) ? 24 : dt == kBf16E && !gated ? 21 : 18;
  const int cap2 = gated && lpr > 64 ? 9 : 8;  // two waves per SIMD
  const bool fits = bwd_waves_per_eu(vpl) == 1 ? vpl <= 9 && streams * vpl <= cap : streams * vpl <= cap2;
  const bool idle = lpr > 64 || (lpr == 64 && bwd_waves_per_eu(vpl) == 1);
  return idle && fits;
}
// Rows over 4 waves at one wave per SIMD that do not fit two register sets
// (longer rows, more input streams) still load the next step early, into
// the registers this step's second pass frees: once a vector's dx is
// stored, that vector's loads of the next step are issued into the
// registers that held it, so the next row streams in while this row's
// second pass computes and stores. Same box, us per 256 MiB of x, cache
// evicted, against loading each step after the last one's stores: D =
// 28672 194.9 -> 175.6, 32768 187.0 -> 172.2, 20002 188.3 -> 180.6, 30002
// 210.7 -> 197.1; residual gradient D = 24576 224.0 -> 220.0, 32768 224.3
// -> 217.6; D = 20480-24576 (weights in registers) within 1%. With two
// workgroups per CU (3 or 4 vectors per lane) the other workgroup already
// fills the gaps, and it cost: fused add with the residual-output gradient
// at D = 4100, 248.3 -> 267.9 us.
constexpr bool bwd_roll(int lpr, int vpl, int mode, int dt) {
  return lpr > 64 && bwd_waves_per_eu(vpl) == 1 && !bwd_prefetch(lpr, vpl, mode, dt);
}

// LDS floats the rows kernel needs: the weights when held in LDS (one float4
// pair per vector slot, laid out so that consecutive lanes read consecutive
// 16 bytes) and, after the rows are done, two rows of D floats for the wave
// merge (which reuse the same space).
inline size_t bwd_rows_lds_floats(int D, bool want_part, bool three_inputs) {
  const RowGeom g = bwd_geom(D);
  const size_t w = bwd_lean(g.vpl, three_inputs) ? static_cast<size_t>(g.vpl) * g.lpr * 8 : 0;
  // merge space: 2 rows of Dp = part_stride(D) floats with one wave per
  // row, 1 with two, none with four
  const int wpr = waves_per_row(g.lpr);
  const size_t m =
      want_part ? static_cast<size_t>(part_stride(D)) * (wpr == 1 ? 2 : wpr == 2 ? 1 : 0) : 0;
  return w > m ? w : m;
}

template <int LPR, int VPL, bool MASKED, int MODE, int DT>
__global__ __launch_bounds__(kBlock)
__attribute__((amdgpu_waves_per_eu(bwd_waves_per_eu(VPL))))
void rmsnorm_bwd_rows_kernel(BwdArgs a) {
  constexpr bool ADD = MODE == kBwdAdd || MODE == kBwdAddGres;
  constexpr bool GRES = MODE == kBwdGres || MODE == kBwdAddGres;
  constexpr bool GATED = MODE == kBwdGatedSilu || MODE == kBwdGatedSigmoid;
  constexpr int ACT = MODE == kBwdGatedSigmoid ? kGateSigmoid : kGateSilu;
  constexpr int RPW = rows_per_wave(LPR);
  constexpr int WPR = waves_per_row(LPR);
  constexpr int U = bwd_unroll(LPR, VPL);
  constexpr int ROWS_WAVE = U * RPW;
  constexpr int ROWS_BLOCK = rows_per_block(LPR, U);
  static_assert(WPR == 1 || (U == 1 && VPL >= kBwdMinVplMulti), "multi-wave rows: one row per step");
  constexpr bool LEAN = bwd_lean(VPL, GATED || ADD);
  constexpr bool PREFETCH = bwd_prefetch(LPR, VPL, MODE, DT);
  constexpr bool ROLL = bwd_roll(LPR, VPL, MODE, DT);
  static_assert(!ROLL || (U == 1 && RPW == 1), "rolling loads: one row per wave step");
  extern __shared__ float lds[];

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
  const int Dp = 8 * nv;           // floats per partial row
  const float Df = static_cast<float>(a.D);
  const bool want_part = a.part != nullptr;

  // Weights w_eff = gamma (+1 in fp32 when zero-centred).
  constexpr bool ELEM = elem_dt(DT);
  // Some lanes lack their last group. Rows of any length with a third input
  // (gate or residual) test every vector from 9 vectors per lane on even
  // when no lane lacks one: without those branches the scheduler holds
  // several vectors at once and spills (D = 32767, same box, cache evicted:
  // gated 1526.2 -> 399.8 us, fused add 504.7 -> 308.6; results unchanged).
  constexpr bool MSK = MASKED || (ELEM && (GATED || ADD) && VPL >= 9);
  // rows of any length: a partial last group is read as the row's last 16
  // bytes, except in rows shorter than one group (LPR == 1)
  constexpr bool TAIL = LPR > 1;
  float wreg[LEAN ? 1 : VPL][8];
  float4* const wl4 = reinterpret_cast<float4*>(lds);
  if constexpr (LEAN) {
    // float4 h (0/1) of group c = v*LPR + l goes to slot (2v + h)*LPR + l
    for (int c = threadIdx.x; c < nv; c += kBlock) {
      float w8[8];
      if constexpr (ELEM) {
        weights_group(a.gamma, a.wdt, a.zc, a.D, c, w8);
      } else {
        weights8(a.gamma, a.wdt, c, w8);
        if (a.zc) {
#pragma unroll
          for (int k = 0; k < 8; ++k) w8[k] = w8[k] + 1.0f;
        }
      }
      wl4[((c / LPR) * 2) * LPR + (c % LPR)] = make_float4(w8[0], w8[1], w8[2], w8[3]);
      wl4[((c / LPR) * 2 + 1) * LPR + (c % LPR)] = make_float4(w8[4], w8[5], w8[6], w8[7]);
    }
    __syncthreads();
  } else {
    if constexpr (ELEM) load_weights_any<LPR, (LEAN ? 1 : VPL)>(a.gamma, a.wdt, a.zc, a.D, l, wreg);
    else load_weights<LPR, (LEAN ? 1 : VPL), MASKED>(a.gamma, a.wdt, a.zc, nv, l, wreg);
  }
  // In the lean plan `base` is an opaque zero, so that the LDS reads stay
  // inside the row loop instead of being hoisted into registers.
  auto weights = [&](int base, int v, float (&w8)[8]) {
    if constexpr (LEAN) {
      const float4 p0 = wl4[base + (2 * v) * LPR + l];
      const float4 p1 = wl4[base + (2 * v + 1) * LPR + l];
      w8[0] = p0.x; w8[1] = p0.y; w8[2] = p0.z; w8[3] = p0.w;
      w8[4] = p1.x; w8[5] = p1.y; w8[6] = p1.z; w8[7] = p1.w;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) w8[k] = wreg[LEAN ? 0 : v][k];
    }
  };

  float acc[VPL][8];
#pragma unroll
  for (int v = 0; v < VPL; ++v)
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[v][k] = 0.0f;

  // Chunk k = the groups of S consecutive row blocks (block b = rows
  // [b*ROWS_BLOCK, (b+1)*ROWS_BLOCK)) numbered k, k + K, k + 2K, ...
  // (K = gridDim.x chunks, S = a.group_blocks), taken from the highest block
  // down. With small S all workgroups sweep one narrow front of the batch
  // together, starting at its end, where the rows the forward read last
  // may still sit in the Infinity Cache.
  const int64_t end = a.T;
  const int64_t nblocks = (a.T + ROWS_BLOCK - 1) / ROWS_BLOCK;
  const int64_t S = a.group_blocks;
  const int64_t ngroups = (nblocks + S - 1) / S;
  const int64_t k = blockIdx.x;
  const int64_t K = gridDim.x;
  const int64_t mine_groups = ngroups > k ? (ngroups - 1 - k) / K + 1 : 0;
  // blocks of this chunk: all S blocks of each group except, possibly, the
  // last group of the batch
  const int64_t last_group = k + (mine_groups - 1) * K;
  const int64_t mine = mine_groups == 0 ? 0 : (mine_groups - 1) * S + (nblocks - last_group * S < S ? nblocks - last_group * S : S);

  // Byte offset of this lane's group v (elements [8c, 8c + 8), c = v*LPR + l)
  // within its row group, per tensor. Rows past the chunk's end read as zero
  // (and then contribute nothing) and their stores drop. With 16-byte
  // storage, groups past D get an offset no resource reaches; in rows of any
  // length the last group's elements are checked one by one
  // (`valid`: the row's elements from the group's first on; `last`: only a
  // lane's last group can be partial).
  auto voff = [&](int v, int64_t ld) -> uint32_t {
    const int c = v * LPR + l;
    if (MSK && c >= nv) return kOutOfRange;
    return static_cast<uint32_t>(slot * ld * 2 + 16 * c);
  };
  auto valid = [&](int v) { return a.D - 8 * (v * LPR + l); };
  auto last = [](int v) { return v == VPL - 1; };
  // Lanes without group v. Only a lane's last one can be missing (VPL =
  // ceil(nv / LPR)); the pipelined rows test only that one. The others test
  // every vector: the branches also keep the scheduler from holding several
  // vectors' values at once, and without them their many vectors per lane
  // no longer fit the register file.
  auto absent = [&](int v) {
    return MSK && (!PREFETCH || v == VPL - 1) && v * LPR + l >= nv;
  };

  // One workgroup step's loaded rows (U row groups of each input stream).
  struct StepRegs {
    u32x4 gq[U][VPL], xq[U][VPL];
    u32x4 rres[GRES ? U : 1][GRES ? VPL : 1];  // residual-branch gradient
    u32x4 zq[GATED ? U : 1][GATED ? VPL : 1];   // gate input
    u32x4 hq[ADD ? U : 1][ADD ? VPL : 1];       // fused add: residual input
    float rq[U];
    int64_t step;  // first row of the block
  };
  // The chunk's blocks from the top: its j-th is block jj % S of the
  // chunk's group jj / S (jj = mine - 1 - j; the last group may be short).
  // Walked one block at a time, carrying the quotient and the remainder, so
  // the loop does no division; past the chunk's last block the walk yields
  // `end`, whose rows are empty.
  int64_t walk_left = mine;
  int64_t walk_q = mine > 0 ? (mine - 1) / S : 0;
  int64_t walk_r = mine > 0 ? (mine - 1) % S : 0;
  auto next_step = [&]() -> int64_t {
    const int64_t st = walk_left > 0 ? ((k + walk_q * K) * S + walk_r) * ROWS_BLOCK : end;
    const bool wrap = walk_r == 0;
    walk_r = wrap ? S - 1 : walk_r - 1;
    walk_q = wrap ? walk_q - 1 : walk_q;
    walk_left = walk_left - 1;
    return st;
  };
  // One step's loads. Two forms, chosen per geometry by measurement (same
  // box, us per 256 MiB of x, cache evicted; the other form in brackets):
  //  - x's cache policy fixed for the whole loop (the caller instantiates
  //    the loop once per policy) and each vector's g and x loads issued
  //    together: the pipelined rows (D = 4096 145.5 [147.9]), the rolling
  //    ones and the other 16-byte rows over 4 waves (before the rolling
  //    loads: D = 20480 164.0 [177.1], 24576 171.8 [188.4]);
  //  - x's policy chosen each step (kXRuntime, a wave-uniform branch) and
  //    all g loads before all x loads: every other row (D = 128 156.9
  //    [162.4], 2048 152.8 [155.1]; before the rolling loads also 20002
  //    187.1 [199.9] and 32768 185.0 [198.6]).
  // x (and the fused add's rin, which the forward read too) takes the
  // streaming hint only when it is well past the Infinity Cache; g (and
  // gres, z) always: they are read once.
  constexpr int kXRuntime = -1;
  auto load_step = [&](auto xpol, int64_t step, StepRegs& b) __attribute__((always_inline)) {
    constexpr int XP = decltype(xpol)::value;
    b.step = step;
    auto load_xp = [&](__amdgpu_buffer_rsrc_t r, int64_t ld, u32x4(&dst)[VPL]) __attribute__((always_inline)) {
      if constexpr (XP == kXRuntime) {
        if (a.x_stream) {
#pragma unroll
          for (int v = 0; v < VPL; ++v) dst[v] = load_row8<DT, kLoadStream, TAIL>(r, voff(v, ld), valid(v), last(v));
        } else {
#pragma unroll
          for (int v = 0; v < VPL; ++v) dst[v] = load_row8<DT, kLoadDefault, TAIL>(r, voff(v, ld), valid(v), last(v));
        }
      } else {
#pragma unroll
        for (int v = 0; v < VPL; ++v)
          dst[v] = load_row8<DT, (XP == kXRuntime ? kLoadDefault : XP), TAIL>(r, voff(v, ld), valid(v), last(v));
      }
    };
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t first = step + group * ROWS_WAVE + u * RPW;
      b.rq[u] = buf_load_f32(f32_rsrc(a.rstd, first, end, RPW), 4 * slot);
      const auto rg = rows_rsrc(a.g, first, end, RPW, a.ld_g, a.D);
      const auto rx = rows_rsrc(a.x, first, end, RPW, a.ld_x, a.D);
      if constexpr (XP == kXRuntime) {
#pragma unroll
        for (int v = 0; v < VPL; ++v)
          b.gq[u][v] = load_row8<DT, kLoadStream, TAIL>(rg, voff(v, a.ld_g), valid(v), last(v));
        load_xp(rx, a.ld_x, b.xq[u]);
      } else {
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          b.gq[u][v] = load_row8<DT, kLoadStream, TAIL>(rg, voff(v, a.ld_g), valid(v), last(v));
          b.xq[u][v] = load_row8<DT, (XP == kXRuntime ? kLoadDefault : XP), TAIL>(rx, voff(v, a.ld_x), valid(v), last(v));
        }
      }
      if constexpr (GRES) {
        const auto rgr = rows_rsrc(a.gres, first, end, RPW, a.ld_gres, a.D);
#pragma unroll
        for (int v = 0; v < VPL; ++v)
          b.rres[u][v] = load_row8<DT, kLoadStream, TAIL>(rgr, voff(v, a.ld_gres), valid(v), last(v));
      }
      if constexpr (GATED) {
        const auto rz = rows_rsrc(a.z, first, end, RPW, a.ld_z, a.D);
#pragma unroll
        for (int v = 0; v < VPL; ++v)
          b.zq[u][v] = load_row8<DT, kLoadStream, TAIL>(rz, voff(v, a.ld_z), valid(v), last(v));
      }
      if constexpr (ADD) load_xp(rows_rsrc(a.rin, first, end, RPW, a.ld_rin, a.D), a.ld_rin, b.hq[u]);
    }
  };
  // Rows of the step after this one, for loads issued while this step's
  // second pass runs (multi-wave rows without the two-set pipeline).
  struct NextRows { __amdgpu_buffer_rsrc_t g, x, gr, z, h; };
  auto roll_begin = [&](int64_t nxt, StepRegs& b) __attribute__((always_inline)) {
    const int64_t nfirst = nxt + group * ROWS_WAVE;
    NextRows n;
    b.step = nxt;
    b.rq[0] = buf_load_f32(f32_rsrc(a.rstd, nfirst, end, RPW), 4 * slot);
    n.g = rows_rsrc(a.g, nfirst, end, RPW, a.ld_g, a.D);
    n.x = rows_rsrc(a.x, nfirst, end, RPW, a.ld_x, a.D);
    if constexpr (GRES) n.gr = rows_rsrc(a.gres, nfirst, end, RPW, a.ld_gres, a.D);
    if constexpr (GATED) n.z = rows_rsrc(a.z, nfirst, end, RPW, a.ld_z, a.D);
    if constexpr (ADD) n.h = rows_rsrc(a.rin, nfirst, end, RPW, a.ld_rin, a.D);
    return n;
  };
  auto roll_load = [&](auto xpol, StepRegs& b, const NextRows& n, int v) __attribute__((always_inline)) {
    constexpr int XP = decltype(xpol)::value;
    b.gq[0][v] = load_row8<DT, kLoadStream, TAIL>(n.g, voff(v, a.ld_g), valid(v), last(v));
    b.xq[0][v] = load_row8<DT, XP, TAIL>(n.x, voff(v, a.ld_x), valid(v), last(v));
    if constexpr (GRES) b.rres[0][v] = load_row8<DT, kLoadStream, TAIL>(n.gr, voff(v, a.ld_gres), valid(v), last(v));
    if constexpr (GATED) b.zq[0][v] = load_row8<DT, kLoadStream, TAIL>(n.z, voff(v, a.ld_z), valid(v), last(v));
    if constexpr (ADD) b.hq[0][v] = load_row8<DT, XP, TAIL>(n.h, voff(v, a.ld_rin), valid(v), last(v));
  };
  auto process_step = [&](auto xpol, int64_t step, StepRegs& b, int64_t nxt) __attribute__((always_inline)) {
    // The row's values as fp32: x, or for the fused add h = x + rin (one fp32
    // rounding, as in the forward).
    auto row_values = [&](int u, int v, float (&f)[8]) {
      unpack8<DT>(b.xq[u][v], f);
      if constexpr (ADD) {
        float rf[8];
        unpack8<DT>(b.hq[u][v], rf);
#pragma unroll
        for (int k = 0; k < 8; ++k) f[k] = f[k] + rf[k];
      }
    };
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t first = step + group * ROWS_WAVE + u * RPW;
      const float r = b.rq[u];
      int wbase = 0;
      if constexpr (LEAN) asm("" : "+v"(wbase));
      // Pass 1: the lane partial of s = sum_i (g_i * w_i) * x_i in (vector,
      // element) order, and this row's (g*x)*r added to the dgamma
      // accumulators (rows past the chunk read as zeros with r = 0 and add
      // +0). Gated: g is first replaced by gn = g * a(z), and
      // dz = (g * ((x * r) * w)) * a'(z) is stored.
      [[maybe_unused]] const auto rdz =
          rows_rsrc(GATED ? a.dz : nullptr, first, GATED && a.dz != nullptr ? end : first, RPW,
                    a.ld_dz, a.D);
      acc_t sa = 0;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        // Lanes without this vector (weights unset) skip its arithmetic. Its
        // stores stay outside the branch, at an offset no resource reaches,
        // so every lane issues the same memory operations: a store count
        // that differed between the branch's paths would leave the compiler
        // unsure how many are in flight, and it would then wait for the next
        // step's loads as well.
        const bool have = !absent(v);
        // A partial last group read as the row's last 16 bytes moves into
        // place here, where it is first used (and stays placed for pass 2).
        // Placed at the top of the step instead, the shifts would stand right
        // after the next step's loads and the compiler would make them wait
        // for part of those loads.
        if (v == VPL - 1) {
          const int lv = valid(VPL - 1);
          place_row8<DT, TAIL>(b.gq[u][VPL - 1], lv, true);
          place_row8<DT, TAIL>(b.xq[u][VPL - 1], lv, true);
          if constexpr (GATED) place_row8<DT, TAIL>(b.zq[u][VPL - 1], lv, true);
          if constexpr (ADD) place_row8<DT, TAIL>(b.hq[u][VPL - 1], lv, true);
        }
        [[maybe_unused]] float dz8[8];
        if constexpr (GATED) {
#pragma unroll
          for (int k = 0; k < 8; ++k) dz8[k] = 0.0f;
        }
        if (have) {
          float gf[8], xf[8], w8[8];
          unpack8<DT>(b.gq[u][v], gf);
          row_values(u, v, xf);
          weights(wbase, v, w8);
          if constexpr (GATED) {
            float zf[8];
            unpack8<DT>(b.zq[u][v], zf);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              float ag, dag;
              gate_and_grad<ACT>(zf[k], ag, dag);
              const float xr = xf[k] * r;
              const float nw = xr * w8[k];
              const float gnw = gf[k] * nw;
              dz8[k] = gnw * dag;
              gf[k] = gf[k] * ag;
            }
          }
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float gw = gf[k] * w8[k];
            const float t = gw * xf[k];
            sa = acc_add(sa, t);
            acc[v][k] = __builtin_fmaf(gf[k] * xf[k], r, acc[v][k]);
          }
        }
        if constexpr (GATED) store_row8<DT>(pack8<DT>(dz8), rdz, voff(v, a.ld_dz), valid(v), last(v));
        // one vector at a time: without this fence the scheduler unpacks the
        // whole row up front and the kernel runs ~10% slower (measured)
        __builtin_amdgcn_sched_barrier(0);
      }
      const float s = static_cast<float>(row_total<LPR>(sa, xch, xstep));
      const float rr = r * r;
      const float r3 = rr * r;
      const float r3s = r3 * s;
      const float c = r3s / Df;
      // Pass 2: dx = gw*r - x*c (+ gres), one rounding to bf16.
      if constexpr (LEAN) {
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          opaque(b.gq[u][v]);
          opaque(b.xq[u][v]);
          if constexpr (GATED) opaque(b.zq[u][v]);
          if constexpr (ADD) opaque(b.hq[u][v]);
        }
        asm("" : "+v"(wbase));
      }
      // Without dx (weight gradient only) the resource is empty and the
      // stores drop; computing dx anyway keeps this loop free of branches.
      const auto rdx = rows_rsrc(a.dx, first, a.dx != nullptr ? end : first, RPW, a.ld_dx, a.D);
      [[maybe_unused]] NextRows nr;
      if constexpr (ROLL) nr = roll_begin(nxt, b);
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const bool have = !absent(v);
        if constexpr (GRES) {
          if (v == VPL - 1) place_row8<DT, TAIL>(b.rres[u][VPL - 1], valid(VPL - 1), true);
        }
        float o[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = 0.0f;
        if (have) {
          float gf[8], xf[8], w8[8];
          unpack8<DT>(b.gq[u][v], gf);
          row_values(u, v, xf);
          weights(wbase, v, w8);
          if constexpr (GATED) {
            float zf[8];
            unpack8<DT>(b.zq[u][v], zf);
#pragma unroll
            for (int k = 0; k < 8; ++k) gf[k] = gf[k] * gate<ACT>(zf[k]);
          }
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float gw = gf[k] * w8[k];
            const float t1 = gw * r;
            const float t2 = xf[k] * c;
            o[k] = t1 - t2;
          }
          if constexpr (GRES) {
            float rf[8];
            unpack8<DT>(b.rres[u][v], rf);
#pragma unroll
            for (int k = 0; k < 8; ++k) o[k] = o[k] + rf[k];
          }
        }
        store_row8<DT>(pack8<DT>(o), rdx, voff(v, a.ld_dx), valid(v), last(v));
        if constexpr (ROLL) roll_load(xpol, b, nr, v);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  if constexpr (PREFETCH) {
    // Software pipeline over two register sets that swap roles each step
    // (no copy between them: a copy would wait for every outstanding memory
    // operation, the previous step's stores included): the next step's
    // loads are in flight while this step computes. Every load is issued
    // unconditionally: past the chunk's last step the rows start at `end`,
    // so the resources are empty and the loads read zeros without touching
    // memory. A load under a branch would leave the compiler unsure how many
    // operations are in flight where the paths meet, and it would then wait
    // for all of them (the next step's loads included) before using the
    // other set. The loop leaves by `break`, so its back edge carries a
    // single path.
    StepRegs ra, rb;
    // x's policy is fixed for the whole loop: a branch between two forms of
    // the loads inside it would again leave the compiler unsure of the count.
    auto run = [&](auto xpol) __attribute__((always_inline)) {
      if (mine > 0) {
        load_step(xpol, next_step(), ra);
        for (int64_t j = 0;; j += 2) {
          load_step(xpol, next_step(), rb);
          process_step(xpol, ra.step, ra, 0);
          if (j + 1 >= mine) break;
          load_step(xpol, next_step(), ra);
          process_step(xpol, rb.step, rb, 0);
          if (j + 2 >= mine) break;
        }
      }
    };
    if (a.x_stream) run(std::integral_constant<int, kLoadStream>{});
    else run(std::integral_constant<int, kLoadDefault>{});
  } else if constexpr (ROLL) {
    // One register set: pass 2 of each step issues the next step's loads
    // (roll_load), so each step starts with its rows already in flight. As
    // in the two-set pipeline, x's policy is fixed for the whole loop and
    // the loads past the chunk's last step read from empty resources.
    auto run = [&](auto xpol) __attribute__((always_inline)) {
      if (mine > 0) {
        StepRegs cur;
        // the first step's loads in the order pass 2 issues them, each
        // vector's after a store that drops (an empty resource), so that
        // both ways into the loop leave the same operations in flight
        const NextRows n0 = roll_begin(next_step(), cur);
        const auto none = rows_rsrc(a.dx, 0, 0, RPW, a.ld_dx, a.D);
        float zero8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) zero8[e] = 0.0f;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          store_row8<DT>(pack8<DT>(zero8), none, voff(v, a.ld_dx), valid(v), last(v));
          roll_load(xpol, cur, n0, v);
        }
        for (int64_t j = 0;; ++j) {
          const int64_t nxt = next_step();
          process_step(xpol, cur.step, cur, nxt);
          if (j + 1 >= mine) break;
        }
      }
    };
    if (a.x_stream) run(std::integral_constant<int, kLoadStream>{});
    else run(std::integral_constant<int, kLoadDefault>{});
  } else {
    auto run = [&](auto xpol) __attribute__((always_inline)) {
      for (int64_t j = 0; j < mine; ++j) {
        StepRegs cur;
        load_step(xpol, next_step(), cur);
        process_step(xpol, cur.step, cur, 0);
      }
    };
    // the load forms above
    if constexpr (LPR > 64 && !ELEM) {
      if (a.x_stream) run(std::integral_constant<int, kLoadStream>{});
      else run(std::integral_constant<int, kLoadDefault>{});
    } else {
      run(std::integral_constant<int, kXRuntime>{});
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

  // Group v of this lane's accumulators to / from a row of Dp floats: the
  // columns 8c .. 8c+7 of group c = v*LPR + l (Dp = 8 * nv, so a partial last
  // group's columns past D exist and hold zeros).
  auto put = [&](float* row, int v) {
    float* d = row + 8 * (v * LPR + l);
    *reinterpret_cast<float4*>(d) = make_float4(acc[v][0], acc[v][1], acc[v][2], acc[v][3]);
    *reinterpret_cast<float4*>(d + 4) = make_float4(acc[v][4], acc[v][5], acc[v][6], acc[v][7]);
  };
  auto add_from = [&](const float* row, int v) {
    const float* d = row + 8 * (v * LPR + l);
    const float4 p0 = *reinterpret_cast<const float4*>(d);
    const float4 p1 = *reinterpret_cast<const float4*>(d + 4);
    acc[v][0] = acc[v][0] + p0.x; acc[v][1] = acc[v][1] + p0.y;
    acc[v][2] = acc[v][2] + p0.z; acc[v][3] = acc[v][3] + p0.w;
    acc[v][4] = acc[v][4] + p1.x; acc[v][5] = acc[v][5] + p1.y;
    acc[v][6] = acc[v][6] + p1.z; acc[v][7] = acc[v][7] + p1.w;
  };
  // lanes without group v
  auto absent_part = [&](int v) { return MSK && v * LPR + l >= nv; };
  float* const out = a.part + static_cast<int64_t>(blockIdx.x) * Dp;
  const bool writer = slot == 0;

  if constexpr (WPR == 4) {
    // Four waves per row: every wave owns distinct columns.
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      if (absent_part(v)) continue;
      put(out, v);
    }
  } else if constexpr (WPR == 2) {
    // Two waves per row: waves 0 and 2 hold the same columns, as do 1 and 3;
    // w0 + w2 and w1 + w3 through one LDS row of Dp floats (the weights'
    // space is reused, hence the barrier first).
    __syncthreads();
    if (wave >= 2) {
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        if (absent_part(v)) continue;
        put(lds, v);
      }
    }
    __syncthreads();
    if (wave < 2) {
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        if (absent_part(v)) continue;
        add_from(lds, v);
        put(out, v);
      }
    }
  } else {
    // One wave per row: ((w0 + w2) + (w1 + w3)) through two LDS rows of Dp
    // floats (the weights' space is reused, hence the barrier first).
    __syncthreads();
    auto lds_row = [&](int b) { return lds + b * Dp; };
    if (wave >= 2 && writer) {
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        if (absent_part(v)) continue;
        put(lds_row(wave - 2), v);
      }
    }
    __syncthreads();
    if (wave < 2 && writer) {
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        if (absent_part(v)) continue;
        add_from(lds_row(wave), v);
        if (wave == 1) put(lds_row(wave), v);  // the same wave read this row just above
      }
    }
    __syncthreads();
    if (wave == 0 && writer) {
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        if (absent_part(v)) continue;
        add_from(lds_row(1), v);
        put(out, v);
      }
    }
  }
}

namespace bwd_detail {

template <int LPR, int VPL, bool MASKED, int MODE, int DT>
int launch_inst(const BwdArgs& a, void* stream) {
  constexpr bool THREE = MODE == kBwdGatedSilu || MODE == kBwdGatedSigmoid || MODE == kBwdAdd ||
                         MODE == kBwdAddGres;
  const size_t lds = sizeof(float) * bwd_rows_lds_floats(a.D, a.part != nullptr, THREE);
  // Rows past 8192 elements may need more than 64 KiB of LDS (at most
  // 128 KiB, within gfx950's 160 KiB): raise the kernel's limit once.
  if (lds > 64 * 1024) {
    static const int lds_ok = [] {
      return static_cast<int>(hipFuncSetAttribute(
          reinterpret_cast<const void*>(&rmsnorm_bwd_rows_kernel<LPR, VPL, MASKED, MODE, DT>),
          hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024));
    }();
    if (lds_ok != 0) return lds_ok;
  }
  hipLaunchKernelGGL((rmsnorm_bwd_rows_kernel<LPR, VPL, MASKED, MODE, DT>),
                     dim3(static_cast<unsigned>(a.chunks)), dim3(kBlock), lds,
                     static_cast<hipStream_t>(stream), a);
  return static_cast<int>(hipGetLastError());
}

using RowsLaunch = int (*)(const BwdArgs&, void*);

template <int MODE, int DT, int VPL = 1>
RowsLaunch pick_wide(int vpl, bool masked) {
  if constexpr (VPL > kMaxVpl) {
    return nullptr;
  } else {
    if (vpl == VPL)
      return masked ? &launch_inst<64, VPL, true, MODE, DT> : &launch_inst<64, VPL, false, MODE, DT>;
    return pick_wide<MODE, DT, VPL + 1>(vpl, masked);
  }
}

// Rows over 4 waves (D > 4096): 3 to 16 vectors per lane.
template <int MODE, int DT, int LPR, int VPL = kBwdMinVplMulti>
RowsLaunch pick_multi(int vpl, bool masked) {
  if constexpr (VPL > kMaxVpl) {
    return nullptr;
  } else {
    if (vpl == VPL)
      return masked ? &launch_inst<LPR, VPL, true, MODE, DT> : &launch_inst<LPR, VPL, false, MODE, DT>;
    return pick_multi<MODE, DT, LPR, VPL + 1>(vpl, masked);
  }
}

template <int MODE, int DT = kBf16>
RowsLaunch pick(const RowGeom& g) {
  switch (g.lpr) {
    case 256: return pick_multi<MODE, DT, 256>(g.vpl, g.masked);
    case 64: return pick_wide<MODE, DT>(g.vpl, g.masked);
    case 32: return g.masked ? &launch_inst<32, 1, true, MODE, DT> : &launch_inst<32, 1, false, MODE, DT>;
    case 16: return g.masked ? &launch_inst<16, 1, true, MODE, DT> : &launch_inst<16, 1, false, MODE, DT>;
    case 8: return g.masked ? &launch_inst<8, 1, true, MODE, DT> : &launch_inst<8, 1, false, MODE, DT>;
    case 4: return g.masked ? &launch_inst<4, 1, true, MODE, DT> : &launch_inst<4, 1, false, MODE, DT>;
    case 2: return &launch_inst<2, 1, false, MODE, DT>;
    case 1: return &launch_inst<1, 1, false, MODE, DT>;
    default: return nullptr;
  }
}

}  // namespace bwd_detail
}  // namespace rmsn
