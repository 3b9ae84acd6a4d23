// Row geometry of the gfx950 kernels, shared by the host launchers and the
// kernels. Everything here is a function of D alone: the batch size, a row's
// index and the row strides never enter, which is what makes each row's
// arithmetic identical in every batch (TransformerEngine issue "Expose Batch
// Invariant Kernels", sections 2-3: the reduction layout must come from the
// problem's fixed dimensions, never from the batch dimension).
//
// A row of D bf16 values is NV = ceil(D/8) groups of 8 consecutive elements
// (16-byte vectors; when D is not a multiple of 8 the last group is
// partial), shared by LPR lanes:
//  - long rows span several wavefronts of one workgroup: LPR = 128 or 256
//    (VPL = ceil(NV/LPR) <= 16 vectors each). Both kernels do this past 512
//    vectors (D > 4096): the forward over 2 waves up to 1024 vectors and 4
//    beyond, the backward always over 4 waves (fwd_geom, bwd_geom); both
//    keep VPL <= 8 up to 2048 vectors (D = 16384);
//  - 64 <= NV: LPR = 64, one wavefront (VPL = ceil(NV/64));
//  - NV < 64: LPR = the smallest power of two >= NV, VPL = 1, and a wave
//    carries 64/LPR rows side by side.
// Lane l of a row (l = 64 * (wave within the row) + lane) owns the vectors
// c = v*LPR + l, v = 0..VPL-1; MASKED marks geometries where the last of
// those vectors is missing on some lanes.
#pragma once

#include <stdint.h>

namespace rmsn {

constexpr int kWaves = 4;            // wavefronts per workgroup
constexpr int kBlock = 64 * kWaves;  // threads per workgroup
constexpr int kMaxD = 32768;
constexpr int kMaxVpl = 16;      // vectors per lane, in every geometry
// Vectors per lane of multi-wave rows: forward 5..16, backward 3..16.
constexpr int kFwdMinVplMulti = 5;
constexpr int kBwdMinVplMulti = 3;
// The backward splits the batch into at most kCus * (its occupancy in
// workgroups per CU) chunks of rows, one workgroup per chunk. Rows of 5 or
// more vectors per lane use the whole register file (one workgroup per CU);
// narrower rows run two per CU, which measured faster (D = 128: 124 us
// instead of 161 us per 256 MiB step), while two per CU at D >= 4096 was
// slower.
constexpr int64_t kCus = 256;
constexpr int bwd_waves_per_eu(int vpl) { return vpl < 5 ? 2 : 1; }
constexpr int64_t kMaxChunks = 2 * kCus;

struct RowGeom {
  int lpr;     // lanes per row (1, 2, 4, ..., 64, 128, 256)
  int vpl;     // 16-byte vectors per lane (1..16)
  bool masked; // some lanes lack their last vector
};

// Wavefronts that share one row, and rows side by side in one wavefront.
constexpr int waves_per_row(int lpr) { return lpr > 64 ? lpr / 64 : 1; }
constexpr int rows_per_wave(int lpr) { return lpr >= 64 ? 1 : 64 / lpr; }

// One wave or fewer per row (NV <= 1024).
inline RowGeom single_wave_geom(int64_t nv) {
  if (nv >= 64) return {64, static_cast<int>((nv + 63) / 64), (nv % 64) != 0};
  int lpr = 1;
  while (lpr < nv) lpr <<= 1;
  return {lpr, 1, lpr != nv};
}

inline RowGeom multi_wave_geom(int64_t nv, int lpr) {
  return {lpr, static_cast<int>((nv + lpr - 1) / lpr), (nv % lpr) != 0};
}

// Forward: past 512 vectors (D > 4096), 2 waves per row up to 1024 vectors,
// 4 beyond, so a lane holds at most 8 vectors up to D = 16384 and the
// kernel keeps 4 waves per SIMD (its weights stay in registers). Against one
// wave per row up to 1024 vectors and 2 up to 2048 (us per 256 MiB of x,
// cache evicted, same box): D = 5120 98.8 -> 95.6, 6144 105.1 -> 95.9, 8192
// 108.0 -> 101.6, 10240 109.2 -> 101.8, 12288 103.0 -> 102.2, 16384 104.6
// -> 101.3; D = 4104 101.3 -> 102.0 (warm 94.3 -> 89.0).
inline RowGeom fwd_geom(int64_t D) {
  const int64_t nv = (D + 7) / 8;
  if (nv > 512) return multi_wave_geom(nv, nv <= 1024 ? 128 : 256);
  return single_wave_geom(nv);
}

// Backward: past 512 vectors (D > 4096), 4 waves per row. Measured on the
// rows kernel per 256 MiB of x against one wave per row (2 waves past 8192):
// D = 8192 147 -> 124 us, 12288 163 -> 132, 16384 168 -> 134 (the software
// pipeline needs VPL <= 9 to fit the register file); D = 5120 within 2%.
inline RowGeom bwd_geom(int64_t D) {
  const int64_t nv = (D + 7) / 8;
  if (nv > 512) return multi_wave_geom(nv, 256);
  return single_wave_geom(nv);
}

// Floats per row of the backward's dgamma partials (and of its LDS merge
// rows): D rounded up to whole groups of 8.
constexpr int64_t part_stride(int64_t D) { return (D + 7) / 8 * 8; }

// Rows a wave keeps in flight per step: enough that each lane has about
// 128 bytes of one input stream outstanding.
#ifndef RMSN_FWD_UNROLL_NARROW
#define RMSN_FWD_UNROLL_NARROW 2
#endif
// Infinity Cache (MALL) capacity of an MI355X. Both kernels read x with the
// non-temporal hint only when x is well past this (the threshold is in
// api.cpp): up to about twice the capacity the backward still finds enough
// of x in the cache (the forward just read it) to pay for keeping its lines;
// beyond that they would only evict other lines. The hint changes no result.
constexpr int64_t kCacheBytes = int64_t{256} << 20;

constexpr int fwd_unroll(int lpr, int vpl) {
  return lpr < 64 ? RMSN_FWD_UNROLL_NARROW
                  : lpr > 64 ? 1 : (vpl == 1 ? 8 : vpl == 2 ? 4 : vpl <= 4 ? 2 : 1);
}
static_assert(RMSN_FWD_UNROLL_NARROW >= 1, "unroll");
#ifndef RMSN_BWD_UNROLL_NARROW
#define RMSN_BWD_UNROLL_NARROW 4
#endif
constexpr int bwd_unroll(int lpr, int vpl) {
  return lpr < 64 ? RMSN_BWD_UNROLL_NARROW : lpr > 64 ? 1 : (vpl == 1 ? 4 : vpl == 2 ? 2 : 1);
}

// Rows one workgroup step covers: (waves / waves per row) row groups of
// U unrolled steps of rows_per_wave rows.
constexpr int rows_per_block(int lpr, int unroll) {
  return kWaves / waves_per_row(lpr) * unroll * rows_per_wave(lpr);
}

inline int64_t bwd_rows_per_step(int64_t D) {
  const RowGeom g = bwd_geom(D);
  return rows_per_block(g.lpr, bwd_unroll(g.lpr, g.vpl));
}

}  // namespace rmsn
