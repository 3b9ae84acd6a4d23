// The backward's dgamma chunk plan (host only: api.cpp computes it and
// passes chunks and group size to the rows kernel as arguments).
#pragma once

#include <stdint.h>

#include "geometry.hpp"

namespace rmsn {

// Row blocks per group of the backward's traversal (0: one contiguous group
// per chunk), where the batch size does not pick it (below). Groups of 4
// blocks keep the workgroups on a front of 256 x 4 blocks.
#ifndef RMSN_BWD_GROUP
#define RMSN_BWD_GROUP 4
#endif

// dgamma chunking for a batch of T rows. The batch is cut into blocks of
// R = bwd_rows_per_step(D) rows (block b = rows [b*R, min(T, (b+1)*R))) and
// the blocks into groups of S consecutive blocks; chunk k of K holds the
// groups k, k+K, k+2K, ... (dgamma sums over the whole batch, so its
// grouping may depend on T; the per-row outputs never do.)
struct BwdPlan {
  int64_t block_rows;    // R
  int64_t chunks;        // K <= kMaxChunks
  int64_t group_blocks;  // S
};

#ifndef RMSN_BWD_BLOCKS_PER_CU
#define RMSN_BWD_BLOCKS_PER_CU 0  // 0: the kernel's occupancy
#endif
inline int64_t bwd_target_chunks(int64_t D) {
  return kCus * (RMSN_BWD_BLOCKS_PER_CU > 0 ? RMSN_BWD_BLOCKS_PER_CU
                                            : bwd_waves_per_eu(bwd_geom(D).vpl));
}

// Rows of one wave with 5 to 8 groups per lane (2048 < D <= 4096) run one
// workgroup per CU and take their (K, S) from measurement
// (rows kernel, cache flushed before each launch, us; after the forward in
// brackets):
//   D     T        K=256 S=4      K=256 S=1      K=512 S=8
//   2560  32768    95.1 ( 82.0)   88.0 ( 78.9)  101.8 ( 79.3)
//   3072  65536   222.0          211.3          238.4
//   3584  131072  526.2          501.4          551.4
//   4096  32768   154.6 (123.8)  149.2 (121.2)  153.1 (126.6)
//   4096  65536   293.6          300.9          288.2
//   4096  131072  588.4          592.4          564.5
//   4096  262144 1186.4         1222.4         1115.2
// Single-block groups dealt over one chunk per CU sweep the batch on one
// dense front; rows of a power-of-two byte length past 32 blocks per CU
// (there a chunk's consecutive blocks lie a power of two apart, 8 MiB of
// each input at D = 4096) take 512 chunks of groups of 8 blocks instead,
// two rounds of workgroups, so the last chunks go to whichever CUs are free.
constexpr int64_t kBwdDenseBlocksPerCu = 32;

inline BwdPlan bwd_plan(int64_t T, int64_t D) {
  const int64_t R = bwd_rows_per_step(D);
  int64_t target = bwd_target_chunks(D);
  if (T <= 0) return {R, 0, 1};
  // ceil divisions written so that no T up to INT64_MAX overflows
  const int64_t blocks = T / R + (T % R != 0);
  int64_t S = RMSN_BWD_GROUP > 0 ? RMSN_BWD_GROUP : blocks / target + (blocks % target != 0);
  const RowGeom g = bwd_geom(D);
  if (RMSN_BWD_GROUP > 0 && RMSN_BWD_BLOCKS_PER_CU == 0 && g.lpr == 64 && g.vpl >= 5) {
    const bool pow2 = (D & (D - 1)) == 0;
    const bool spread = pow2 && blocks > kBwdDenseBlocksPerCu * kCus;
    S = spread ? 8 : 1;
    target = spread ? 2 * kCus : kCus;
  }
  const int64_t groups = blocks / S + (blocks % S != 0);
  return {R, groups < target ? groups : target, S};
}

}  // namespace rmsn
