// Batch-invariant BF16 GEMM Y = X @ W.T on gfx950 matrix cores.
//
// TransformerEngine issue "Expose Batch Invariant Kernels", point 3: the
// library GEMM was not batch-invariant because the algorithm (and with it
// the reduction order) was chosen from the whole problem shape; a GEMM whose
// output tiles accumulate over K in a fixed BLOCK_K loop, with no split-K, is
// invariant. What fixes an output element's value here is its arithmetic
// alone: an fp32 accumulator that starts at zero and takes one
// v_mfma_f32_32x32x16_bf16 step per 16 consecutive k, in ascending k, then
// one rounding to bf16. Every tile instance below does exactly that for
// every element, so the tile shape (which may follow M and N) changes which
// workgroup computes an element, never how.
//
// The kernel is a template over its tile: TM x TN MFMA blocks of 32 x 32
// per wave, WGM x WGN waves per workgroup, so a workgroup owns
// BM = 32 TM WGM rows by BN = 32 TN WGN columns; K in stages of 64. The
// operands go from memory straight into LDS (buffer loads with the LDS bit:
// lane i's 16 bytes land 16 i bytes past the wave's LDS pointer), through a
// ring of NS stage buffers with one barrier per stage. Rows of X past M and
// rows of W past N read as zero (buffer resources), outputs past M or N are
// not stored, and in a last stage of 32 valid k (K = 32 mod 64) the MFMA
// steps past K are skipped.
// X [M, K] and W [N, K] are row-major with K contiguous: MFMA lane l takes
// 8 consecutive k of row l % 32 at k-offset 8 * (l / 32) for both operands,
// and holds output rows 8 * (r / 4) + 4 * (l / 32) + r % 4 (r = 0..15) of
// column l % 32.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace rmsn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Tile (tm, tn) of workgroup b. Workgroups go to the 8 XCDs round-robin
// (b mod 8); consecutive tiles are given to one XCD, and tiles are numbered
// in groups of kGroupM tile rows, column by column within a group, so the
// tiles an XCD runs at one time share few rows of X and of W in its L2.
#ifndef RMSN_GEMM_XCDS
#define RMSN_GEMM_XCDS 8
#endif
#ifndef RMSN_GEMM_GROUP_M
#define RMSN_GEMM_GROUP_M 4
#endif
constexpr int kXcds = RMSN_GEMM_XCDS, kGroupM = RMSN_GEMM_GROUP_M;
__device__ __forceinline__ void tile_of(int64_t b, int64_t tiles_m, int64_t tiles_n, int64_t& tm,
                                        int64_t& tn) {
  const int64_t P = tiles_m * tiles_n;
  const int64_t xcd = b % kXcds, j = b / kXcds;
  const int64_t per = (P + kXcds - 1) / kXcds;
  const int64_t tall = P % kXcds == 0 ? kXcds : P % kXcds;  // XCDs that take `per` tiles
  const int64_t t = xcd < tall ? xcd * per + j : tall * per + (xcd - tall) * (per - 1) + j;
  const int64_t in_group = kGroupM * tiles_n;
  const int64_t first_m = (t / in_group) * kGroupM;
  const int64_t rows = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
  tm = first_m + (t % in_group) % rows;
  tn = (t % in_group) / rows;
}

// 16 bytes per lane from a buffer resource into LDS: lane i's bytes land at
// lds + 16 i (lds is wave-uniform; it becomes M0).
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, 0, 0, 0);
}

// s_waitcnt vmcnt(N), not waiting on the other counters (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 = 7, lgkmcnt 11:8 = 15).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
// Waits until at most `stages` stages of LPS loads each are in flight (K:
// the most there can be).
template <int LPS, int K>
__device__ __forceinline__ void wait_stages(int stages) {
  if constexpr (K <= 0) {
    wait_vmcnt<0>();
  } else {
    if (stages >= K) {
      wait_vmcnt<K * LPS>();
      return;
    }
    wait_stages<LPS, K - 1>(stages);
  }
}

// 16-byte chunk of a stage row that holds logical chunk kc of row r: kc xor
// swz(r). With 128-byte stage rows (BK = 64) it makes the fragment reads
// (rows r .. r + 15 of one chunk per 16 lanes) hit 16 different 16-byte bank
// groups, and also the 8-lane groups of a 32-bank LDS; the 8 lanes that load
// one row still cover its 128 bytes.
__device__ __forceinline__ int stage_swizzle(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Stage layout: A rows (BM x 128 bytes), then B rows (BN x 128 bytes), no
// padding. Load j of wave w fills 1 KB block w * L + j of a region: row
// 8 * block + lane / 8, physical chunk lane % 8. Loads run NS - 1 stages
// ahead: the barrier before a stage's last k-step makes the next stage
// complete (every wave waited for its own loads) and this stage's buffer
// free (every wave waited for its own fragment reads), the buffer is
// refilled with stage kt + NS, and the next stage's first fragments are read
// while the last k-step's products run.
template <int TM, int TN, int WGM, int WGN, int NS>
__global__ __launch_bounds__(64 * WGM * WGN) void bigemm_dl_kernel(GemmArgs a) {
  constexpr int BK = 64, S = BK / 16, ROWB = 2 * BK;
  constexpr int NW = WGM * WGN;
  constexpr int BM = 32 * TM * WGM, BN = 32 * TN * WGN;
  constexpr int SA = BM * ROWB, STAGE = (BM + BN) * ROWB;
  constexpr int LA = SA / 1024 / NW, LB = BN * ROWB / 1024 / NW;  // 1 KB loads per wave
  constexpr int LPS = LA + LB;
  static_assert(LA * 1024 * NW == SA && LB * 1024 * NW == BN * ROWB, "whole 1 KB loads per wave");
  static_assert((NS - 1) * LPS < 64, "loads in flight fit the vmcnt counter");
  extern __shared__ __attribute__((aligned(16))) char lds8[];

  int64_t tm, tn;
  tile_of(blockIdx.x, (a.M + BM - 1) / BM, (a.N + BN - 1) / BN, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wm = wave / WGN, wn = wave % WGN;
  const int K = static_cast<int>(a.K);
  const auto rx = rows_rsrc(a.x, m0, a.M, BM, a.ld_x, K);
  const auto rw = rows_rsrc(a.w, n0, a.N, BN, a.ld_w, K);

  uint32_t offa[LA], offb[LB];
#pragma unroll
  for (int j = 0; j < LA; ++j) {
    const int row = 8 * (wave * LA + j) + lane / 8;
    offa[j] = static_cast<uint32_t>((row * a.ld_x + 8 * ((lane % 8) ^ stage_swizzle(row))) * 2);
  }
#pragma unroll
  for (int j = 0; j < LB; ++j) {
    const int row = 8 * (wave * LB + j) + lane / 8;
    offb[j] = static_cast<uint32_t>((row * a.ld_w + 8 * ((lane % 8) ^ stage_swizzle(row))) * 2);
  }
  auto issue = [&](int kt, int buf) {
    char* base = lds8 + buf * STAGE;
    const uint32_t kb = static_cast<uint32_t>(kt * BK * 2);
#pragma unroll
    for (int j = 0; j < LA; ++j) load_lds16(rx, base + (wave * LA + j) * 1024, offa[j] + kb);
#pragma unroll
    for (int j = 0; j < LB; ++j) load_lds16(rw, base + SA + (wave * LB + j) * 1024, offb[j] + kb);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  // Fragments of k-step s: A rows wm*32*TM + 32 i + (lane & 31), B rows
  // wn*32*TN + 32 j + (lane & 31), logical chunk 2 s + (lane >> 5); row & 15
  // equals lane & 15, so the swizzle is the lane's own.
  const int sw = stage_swizzle(lane & 31);
  const int arow = (wm * 32 * TM + (lane & 31)) * ROWB;
  const int brow = SA + (wn * 32 * TN + (lane & 31)) * ROWB;
  struct Frags {
    bf16x8 a[TM], b[TN];
  };
  // read in the order the products use them: a0, b0 .. b(TN-1), a1 ..
  auto read_frags = [&](Frags& f, int buf, int s) {
    const char* base = lds8 + buf * STAGE + 16 * ((2 * s + (lane >> 5)) ^ sw);
    f.a[0] = *reinterpret_cast<const bf16x8*>(base + arow);
#pragma unroll
    for (int j = 0; j < TN; ++j) f.b[j] = *reinterpret_cast<const bf16x8*>(base + brow + 32 * j * ROWB);
#pragma unroll
    for (int i = 1; i < TM; ++i) f.a[i] = *reinterpret_cast<const bf16x8*>(base + arow + 32 * i * ROWB);
  };
  auto mfma = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
  };
  // A k-step's order: the next step's fragment reads spread over its
  // products, nothing moved across steps (without it the scheduler pulls
  // each read next to the product that needs it and waits on it there).
  auto pin_step = [&]() {
    constexpr int PER = TM * TN / (TM + TN) > 0 ? TM * TN / (TM + TN) : 1;
#pragma unroll
    for (int q = 0; q < TM + TN; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);  // then PER products
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  const int nk = (K + BK - 1) / BK;
  const int last_steps = (K - (nk - 1) * BK) / 16;  // 4, or 2 when K = 32 mod 64
#pragma unroll
  for (int j = 0; j < NS; ++j)
    if (j < nk) issue(j, j);
  wait_stages<LPS, NS - 1>(nk - 1 < NS - 1 ? nk - 1 : NS - 1);  // stage 0 complete
  __syncthreads();
  Frags f[2];
  read_frags(f[0], 0, 0);
  for (int kt = 0; kt + 1 < nk; ++kt) {
    const int buf = kt % NS;
#pragma unroll
    for (int s = 0; s + 1 < S; ++s) {
      read_frags(f[(s + 1) & 1], buf, s + 1);
      mfma(f[s & 1]);
      pin_step();
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this stage's reads are done
    wait_stages<LPS, NS - 2>(nk - 2 - kt < NS - 2 ? nk - 2 - kt : NS - 2);  // stage kt + 1 complete
    __syncthreads();
    if (kt + NS < nk) issue(kt + NS, buf);
    __builtin_amdgcn_sched_barrier(0);
    read_frags(f[S & 1], (kt + 1) % NS, 0);
    mfma(f[(S - 1) & 1]);
    pin_step();
  }
  {
    const int buf = (nk - 1) % NS;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (s >= last_steps) break;
      if (s + 1 < S && s + 1 < last_steps) read_frags(f[(s + 1) & 1], buf, s + 1);
      mfma(f[s & 1]);
    }
  }

  // Epilogue: each fp32 sum rounded once to bf16; lanes 0..31 store 32
  // consecutive columns of one row, lanes 32..63 the same columns 4 rows on.
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t col = n0 + wn * 32 * TN + 32 * j + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 32 * TM + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < a.M && col < a.N)
          a.y[row * a.ld_y + col] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[i][j][r]));
      }
    }
}

template <int TM, int TN, int WGM, int WGN, int NS>
int launch_dl_tile(const GemmArgs& a, void* stream) {
  constexpr int BM = 32 * TM * WGM, BN = 32 * TN * WGN;
  constexpr int kLds = NS * (BM + BN) * 64 * 2;
  auto* kern = &bigemm_dl_kernel<TM, TN, WGM, WGN, NS>;
  if (kLds > 64 * 1024) {
    static const int lds_ok = [kern] {
      return static_cast<int>(hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, kLds));
    }();
    if (lds_ok != 0) return lds_ok;
  }
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(tiles)), dim3(64 * WGM * WGN), kLds,
                     static_cast<hipStream_t>(stream), a);
  return static_cast<int>(hipGetLastError());
}

// The tiles, largest first: (TM, TN, WGM, WGN), stages NS, LDS.
//   256 x 256: 8 waves of 128 x 64, 2 stages (128 KiB)
//   128 x 256: 8 waves of 64 x 64, 2 stages (96 KiB)
//   128 x 128: 4 waves of 64 x 64, 3 stages (96 KiB)
//   64 x 128: 4 waves of 32 x 64, 4 stages (96 KiB)
//   32 x 64: 2 waves of 32 x 32, 4 stages (48 KiB)
// A launch takes the tile with the least estimated time: rounds of tiles
// over the compute units, ceil(tiles / kCus), times the tile's measured
// time per round at K = 4096 (the same for any K up to a factor, so the
// choice does not depend on K); ties go to the larger tile. The small
// tiles run their K loop at a latency-bound pace that barely shrinks with
// the tile, so a round of bigger tiles often beats more rounds of smaller
// ones. Per-round times, and the launches they give (us at N = K = 4096,
// medians of interleaved timings; the library GEMM in brackets): 256x256
// 113.8 (M = 4096), 128x256 64.0 (M = 2048), 128x128 39.6 (M = 1024),
// 64x128 25.8 (M = 512: 26.5 [26.0]; M = 300: 24.3 [21.7]), 32x64 19.4
// (M = 1: 19.3 [19.2]; M = 128: 20.2 [20.1]).
struct TileInfo {
  int bm, bn;
  int64_t round_ns;  // time of one round of these tiles at K = 4096
  int (*launch)(const GemmArgs&, void*);
};
constexpr int kTiles = 5;
const TileInfo kTileTable[kTiles] = {
    {256, 256, 113800, &launch_dl_tile<4, 2, 2, 4, 2>},
    {128, 256, 64000, &launch_dl_tile<2, 2, 2, 4, 2>},
    {128, 128, 39600, &launch_dl_tile<2, 2, 2, 2, 3>},
    {64, 128, 25800, &launch_dl_tile<1, 2, 2, 2, 4>},
    {32, 64, 19400, &launch_dl_tile<1, 1, 1, 2, 4>},
};

const TileInfo& pick_tile(int64_t M, int64_t N) {
  int best = kTiles - 1;
  int64_t best_ns = -1;
  for (int i = 0; i < kTiles; ++i) {
    const TileInfo& t = kTileTable[i];
    const int64_t tiles = ((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
    const int64_t rounds = tiles == 0 ? 1 : (tiles + kCus - 1) / kCus;
    // rounds <= 2^31 / 256 (the host bounds the 32 x 64 tile count), so
    // rounds * round_ns stays far below 2^63
    const int64_t ns = rounds * t.round_ns;
    if (best_ns < 0 || ns < best_ns) {
      best = i;
      best_ns = ns;
    }
  }
  return kTileTable[best];
}

}  // namespace

void gemm_tile(int64_t M, int64_t N, int64_t* bm, int64_t* bn) {
  const TileInfo& t = pick_tile(M, N);
  *bm = t.bm;
  *bn = t.bn;
}

int launch_gemm(const GemmArgs& a, void* stream) {
  if (a.M == 0 || a.N == 0) return 0;
  return pick_tile(a.M, a.N).launch(a, stream);
}

}  // namespace rmsn
