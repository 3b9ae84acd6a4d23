// Device helpers for the gfx950 RMSNorm kernels: bf16 widening and
// narrowing, 16-byte vector access, and the fixed within-row reduction tree.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "geometry.hpp"

namespace rmsn {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Storage types (the ABI's RMSN_DTYPE_* values): activations are bf16 or
// fp16, weights bf16, fp16 or fp32.
enum : int { kBf16 = 0, kF16 = 1, kF32 = 2 };
// Row storage of a kernel instance: the activation type, plus kElem when
// rows may have any length D and any 2-byte alignment. Either way a lane's
// group c holds the row's elements [8c, 8c + 8) (the last group of a row of
// D not a multiple of 8 is partial; its elements past D read as zero and are
// never written), so the lanes' elements, and hence every reduction tree,
// are those of 16-byte rows of ceil(D/8) groups.
enum : int { kElem = 8, kBf16E = kBf16 | kElem, kF16E = kF16 | kElem };
constexpr int value_dt(int DT) { return DT & ~kElem; }
constexpr bool elem_dt(int DT) { return (DT & kElem) != 0; }
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Unpack the 8 bf16 values of a 16-byte vector, in memory order.
__device__ __forceinline__ void unpack8(const u32x4& q, float (&f)[8]) {
  f[0] = bf16_lo(q.x); f[1] = bf16_hi(q.x);
  f[2] = bf16_lo(q.y); f[3] = bf16_hi(q.y);
  f[4] = bf16_lo(q.z); f[5] = bf16_hi(q.z);
  f[6] = bf16_lo(q.w); f[7] = bf16_hi(q.w);
}

// fp16 pair -> fp32 pair (exact, v_cvt_f32_f16), the low half first.
__device__ __forceinline__ f32x2 f16_pair(uint32_t w) {
  return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
}

// Unpack 8 activations of storage type DT (kBf16 or kF16, with or without
// kElem).
template <int DT>
__device__ __forceinline__ void unpack8(const u32x4& q, float (&f)[8]) {
  if constexpr (value_dt(DT) == kBf16) {
    unpack8(q, f);
  } else {
    const f32x2 a = f16_pair(q.x), b = f16_pair(q.y), c = f16_pair(q.z), d = f16_pair(q.w);
    f[0] = a.x; f[1] = a.y; f[2] = b.x; f[3] = b.y;
    f[4] = c.x; f[5] = c.y; f[6] = d.x; f[7] = d.y;
  }
}

// fp32 pair -> packed bf16 pair with round-to-nearest-even (one
// v_cvt_pk_bf16_f32 on gfx950); the first value lands in the low half.
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f32x2 v = {a, b};
  const bf16x2 h = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
  return u32x4{pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7])};
}

// fp32 pair -> fp16 pair, round to nearest even (the default rounding mode;
// fp16 subnormals are kept, overflow goes to infinity).
__device__ __forceinline__ uint32_t pack2_f16(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// Pack 8 fp32 values to storage type DT with one rounding each.
template <int DT>
__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
  if constexpr (value_dt(DT) == kBf16) {
    return pack8(f);
  } else {
    return u32x4{pack2_f16(f[0], f[1]), pack2_f16(f[2], f[3]), pack2_f16(f[4], f[5]),
                 pack2_f16(f[6], f[7])};
  }
}

// ---- buffer access -----------------------------------------------------------
// Rows are read and written through buffer resources: a wave-uniform base
// address and byte count in scalar registers plus a 32-bit per-lane offset.
// The hardware returns zeros for loads at or past the byte count and drops
// such stores, so rows past the end of the batch (or of a chunk) and vectors
// past D need no branches: they are given offsets beyond the count.
// Word 3 of the descriptor selects 32-bit raw access on gfx9-family parts.
constexpr uint32_t kBufWord3 = 0x00020000u;
// An offset no resource built below reaches (all counts stay under 2^31).
constexpr uint32_t kOutOfRange = 0x80000000u;

// Resource over the rows [first, min(first + cap, limit)) (empty when
// first >= limit), each row D bf16 values at a stride of ld elements. With
// cap <= 64 and ld <= 2^24 (checked by the host) the byte count stays below
// 2^31.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int64_t first,
                                                            int64_t limit, int cap, int64_t ld,
                                                            int D) {
  const int64_t left = limit - first;
  const int64_t count = left < cap ? left : cap;
  const char* p = static_cast<const char*>(base) + first * ld * 2;
  const uint32_t n = count > 0 ? static_cast<uint32_t>(((count - 1) * ld + D) * 2) : 0u;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), 0, static_cast<int>(n), kBufWord3);
}

// Resource over the fp32 values [first, min(first + cap, limit)).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t f32_rsrc(const float* base, int64_t first,
                                                           int64_t limit, int cap) {
  const int64_t left = limit - first;
  const int64_t count = left < cap ? left : cap;
  const uint32_t n = count > 0 ? static_cast<uint32_t>(count * 4) : 0u;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base + first), 0, static_cast<int>(n),
                                           kBufWord3);
}

// Cache policy of a load: kLoadDefault, or kLoadStream (the non-temporal hint:
// the line is not kept for reuse). Streams read once, and nowhere else in the
// same pass, take the hint.
enum : int { kLoadDefault = 0, kLoadStream = 2 };
template <int POLICY = kLoadDefault>
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, POLICY));
}
// Streaming store (non-temporal: the line is not kept in the caches).
__device__ __forceinline__ void buf_store16_nt(const u32x4& v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>(off), 0, 2);
}

// One lane's group of 8 row elements [8c, 8c + 8) through a row resource, at
// byte offset `off` (the group's first element); `left` = D - 8c, the row's
// elements from there on, and `last` whether the group may be the row's
// last (only the last of a lane's groups can be; the argument is a constant
// after unrolling). 16-byte storage: one aligned 16-byte vector.
// Element-wise storage (any D, any 2-byte alignment): a full group is one
// 16-byte access at a 2-byte-aligned offset, which the hardware splits into
// aligned pieces. The row's partial last group (0 < left < 8) is read as the
// 16 bytes that end at the row's last element, which lie inside the row
// whenever D >= 8 (TAIL), and place_row8 moves its elements into place once
// the data is needed: a single load whose result nothing waits for while
// the step's other loads are in flight. Rows shorter than 8 elements (not
// TAIL) read the group element by element, elements past D reading as zero.
// Groups past the row (left <= 0) read zeros.
template <int DT, int POLICY = kLoadDefault, bool TAIL = true>
__device__ __forceinline__ u32x4 load_row8(__amdgpu_buffer_rsrc_t r, uint32_t off, int left,
                                           bool last) {
  if (!elem_dt(DT) || !last || left >= 8) return buf_load16<POLICY>(r, off);
  if constexpr (TAIL) {
    return buf_load16<POLICY>(r, left > 0 ? off - 2u * static_cast<uint32_t>(8 - left) : kOutOfRange);
  } else {
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      h[e] = __builtin_amdgcn_raw_buffer_load_b16(
          r, static_cast<int>(e < left ? off + 2 * e : kOutOfRange), 0, POLICY);
    return u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
  }
}
// Places a group that load_row8 read as a row's tail: its last `left`
// elements become elements 0 .. left-1, zeros above. Every other group is
// left as it is.
template <int DT, bool TAIL = true>
__device__ __forceinline__ void place_row8(u32x4& q, int left, bool last) {
  if constexpr (elem_dt(DT) && TAIL) {
    if (last && left > 0 && left < 8) {
      const unsigned __int128 w = __builtin_bit_cast(unsigned __int128, q);
      q = __builtin_bit_cast(u32x4, w >> (16 * (8 - left)));
    }
  }
}
// Stores a group the same way (non-temporal); a partial last group writes
// only its elements inside the row. A lane's last group in a row of any
// length goes out as the same four stores on every lane, whatever the group
// holds: one 16-byte store for a full group, and pieces of 8, 4 and 2 bytes
// for a partial one (1..7 elements); the stores a lane does not need get an
// offset no resource reaches. (A number of stores that differed between
// lanes' branches would leave the compiler unsure how many memory operations
// are in flight after them, and it would then wait for loads issued ahead
// for the next rows.)
template <int DT>
__device__ __forceinline__ void store_row8(const u32x4& v, __amdgpu_buffer_rsrc_t r, uint32_t off,
                                           int left, bool last) {
  if (!elem_dt(DT) || !last) {
    buf_store16_nt(v, r, off);
    return;
  }
  const bool part = left > 0 && left < 8;
  buf_store16_nt(v, r, left >= 8 ? off : kOutOfRange);
  // elements 0..3
  const bool p8 = part && left >= 4;
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{v.x, v.y}, r, static_cast<int>(p8 ? off : kOutOfRange), 0, 0);
  // the next two elements, from element b
  const int b = p8 ? 4 : 0;
  const bool p4 = part && left - b >= 2;
  __builtin_amdgcn_raw_buffer_store_b32(p8 ? v.z : v.x, r,
                                        static_cast<int>(p4 ? off + 2 * b : kOutOfRange), 0, 0);
  // an odd count's last element e = left - 1 (even: the low half of word e/2)
  const int e = left - 1;
  const bool p2 = part && (left & 1) != 0;
  const uint32_t we = e >= 4 ? (e >= 6 ? v.w : v.z) : (e >= 2 ? v.y : v.x);
  __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(we & 0xFFFFu), r,
                                        static_cast<int>(p2 ? off + 2 * e : kOutOfRange), 0, 0);
}

__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, 0));
}

// The wave's index within the workgroup, known to the compiler as uniform.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
}

// Makes the compiler treat a register vector as rewritten here, so values it
// derived from the vector earlier (unpacked floats, products) are recomputed
// afterwards instead of being kept alive. Re-deriving them costs one VALU op
// each; keeping them would cost a row's worth of extra registers.
__device__ __forceinline__ void opaque(u32x4& q) { asm("" : "+v"(q)); }

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

// The same butterfly on fp64 partials (each 64-bit value moves as two 32-bit
// halves through the same DPP / swizzle / readlane patterns).
template <int CTRL>
__device__ __forceinline__ double dpp64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(b)), CTRL, 0xF, 0xF, false));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(b >> 32)), CTRL, 0xF, 0xF, false));
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ double swizzle_xor16_64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_ds_swizzle(static_cast<int>(static_cast<uint32_t>(b)), 0x401F));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_ds_swizzle(static_cast<int>(static_cast<uint32_t>(b >> 32)), 0x401F));
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ double readlane64(double v, int lane) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(b)), lane));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(b >> 32)), lane));
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

template <int LPR>
__device__ __forceinline__ double row_sum(double v) {
  if constexpr (LPR >= 2) v = v + dpp64<0xB1>(v);
  if constexpr (LPR >= 4) v = v + dpp64<0x4E>(v);
  if constexpr (LPR >= 8) v = v + dpp64<0x141>(v);
  if constexpr (LPR >= 16) v = v + dpp64<0x140>(v);
  if constexpr (LPR >= 32) v = v + swizzle_xor16_64(v);
  if constexpr (LPR >= 64) v = readlane64(v, 0) + readlane64(v, 32);
  return v;
}

// Sum of v over all LPR lanes of a row, returned to each of them with
// identical bits. Up to 64 lanes this is row_sum. A row spread over W = LPR/64
// wavefronts first reduces within each wave, then adds the W wave totals in
// a fixed tree, (t0 + t1) or ((t0 + t1) + (t2 + t3)), through LDS: `xch`
// holds two buffers of kWaves doubles, used alternately (`step` counts the
// exchanges), so a buffer is rewritten only after every wave has passed the
// next exchange's barrier and hence finished reading it. Every wave of the
// workgroup must make the same sequence of calls (each holds a barrier).
template <int LPR>
__device__ __forceinline__ double row_total(double v, double (*xch)[kWaves], int& step) {
  if constexpr (LPR <= 64) {
    return row_sum<LPR>(v);
  } else {
    constexpr int W = LPR / 64;
    static_assert(W == 2 || W == 4, "rows span 2 or 4 waves");
    const double t = row_sum<64>(v);
    const int wave = wave_id();
    double* b = xch[step & 1];
    ++step;
    b[wave] = t;  // every lane holds t; no branch around the store
    __syncthreads();
    const int first = (wave / W) * W;
    if constexpr (W == 2) return b[first] + b[first + 1];
    else return (b[first] + b[first + 1]) + (b[first + 2] + b[first + 3]);
  }
}

// Row reductions accumulate fp32 terms (squares of bf16 values, which are
// exact, and the fp32 products gw*x) in fp64 along the fixed tree above, and
// round the total to fp32 once. The fp64 sum of such terms is exact, or
// within a few fp64 ulp of exact, whatever the order, so the fp32 result is
// the same as an ordered sum's except when the exact value lies within those
// few fp64 ulp of an fp32 rounding boundary.
typedef double acc_t;
__device__ __forceinline__ acc_t acc_add(acc_t a, float t) { return a + static_cast<acc_t>(t); }

// r = rsqrt(ss / D + eps): the mean is an fp32 division and the sum with eps
// an fp32 addition; the reciprocal square root is 1/sqrt taken in fp64 (both
// operations correctly rounded) and rounded to fp32 once.
__device__ __forceinline__ float rstd_of(float ss, float Df, float eps) {
  const float mean = ss / Df;
  const float var = mean + eps;
  return static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(var)));
}

// ---- gate activations of the gated norm -----------------------------------
enum : int { kGateSilu = 0, kGateSigmoid = 1 };

// sigmoid(z) and 1 - sigmoid(z), each within a few fp32 ulp, from
// e = exp(-|z|): for z >= 0 they are 1/(1+e) and e/(1+e), for z < 0 the other
// way round, so neither is a cancelling subtraction and nothing overflows.
// exp(-|z|) = 2^y with y = -|z| log2(e) carried in two parts (argument
// splitting after Cody and Waite): y_hi = fp32(-|z| * L) and y_lo = the
// rounding error of that product (an fma) plus -|z| * (log2(e) - L);
// then e = 2^y_hi * (1 + y_lo ln 2). |z| is clamped to 128, far past the
// point where e underflows, so infinities give e = 0; NaN passes through.
// The reciprocal is v_rcp_f32 refined by one Newton step.
__device__ __forceinline__ void sigmoid_pair(float z, float& s, float& sc) {
  constexpr float kL = 1.44269504088896340736f;
  constexpr float kLlo = static_cast<float>(1.44269504088896340736 - static_cast<double>(kL));
  constexpr float kLn2 = 0.69314718055994530942f;
  float m = -__builtin_fabsf(z);
  m = m < -128.0f ? -128.0f : m;
  const float yh = m * kL;
  const float yl = __builtin_fmaf(m, kL, -yh) + m * kLlo;
  const float eh = __builtin_exp2f(yh);  // subnormal results kept
  const float e = __builtin_fmaf(eh, yl * kLn2, eh);
  const float d = 1.0f + e;
  float inv = __builtin_amdgcn_rcpf(d);
  inv = __builtin_fmaf(__builtin_fmaf(-d, inv, 1.0f), inv, inv);
  const float ei = e * inv;
  const bool pos = z >= 0.0f;
  s = pos ? inv : ei;
  sc = pos ? ei : inv;
}

// The gate a(z): silu(z) = z * sigmoid(z), or sigmoid(z).
template <int ACT>
__device__ __forceinline__ float gate(float z) {
  float s, sc;
  sigmoid_pair(z, s, sc);
  return ACT == kGateSigmoid ? s : z * s;
}

// The forward's gate: a(z) to about 2^-16 relative, which keeps a bf16
// output within 1 ulp of the correctly rounded one, at about half the
// instructions of gate() (the forward of a gated norm is otherwise bound by
// its arithmetic). e = exp(-|z|) is 2^(y/2) squared, y = -|z| log2(e): the
// half power is never subnormal, and the square rounds gradually into the
// subnormal range, so the hardware exponential needs no range scaling;
// sigmoid is 1/(1+e) or e/(1+e) by the sign of z (v_rcp_f32, 1 ulp).
// Infinities give e = 0 and NaN passes through, as in gate().
__device__ __forceinline__ float sigmoid_fast(float z) {
  constexpr float kHalfL = 0.72134752044448170368f;  // log2(e) / 2
  const float h = __builtin_amdgcn_exp2f(-__builtin_fabsf(z) * kHalfL);
  const float e = h * h;
  const float inv = __builtin_amdgcn_rcpf(1.0f + e);
  return z >= 0.0f ? inv : e * inv;
}
template <int ACT>
__device__ __forceinline__ float gate_fast(float z) {
  const float s = sigmoid_fast(z);
  return ACT == kGateSigmoid ? s : z * s;
}

// a(z) and a'(z): silu' = s (1 + z (1 - s)), sigmoid' = s (1 - s).
template <int ACT>
__device__ __forceinline__ void gate_and_grad(float z, float& a, float& da) {
  float s, sc;
  sigmoid_pair(z, s, sc);
  if constexpr (ACT == kGateSigmoid) {
    a = s;
    da = s * sc;
  } else {
    a = z * s;
    const float zsc = z * sc;
    da = s * (1.0f + zsc);
  }
}

// Rounds 8 fp32 values to the activation storage type DT and back (round
// to nearest even).
template <int DT>
__device__ __forceinline__ void round8(float (&f)[8]) { unpack8<DT>(pack8<DT>(f), f); }

// The 8 weights of vector c in fp32, widened exactly from their storage
// type `wdt` (the weights are read once per workgroup, so the type is a
// run-time choice).
__device__ __forceinline__ void weights8(const void* __restrict__ gamma, int wdt, int c,
                                         float (&w)[8]) {
  if (wdt == kF32) {
    const float4 a = reinterpret_cast<const float4*>(gamma)[2 * c];
    const float4 b = reinterpret_cast<const float4*>(gamma)[2 * c + 1];
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  } else {
    const u32x4 q = reinterpret_cast<const u32x4*>(gamma)[c];
    if (wdt == kF16) unpack8<kF16>(q, w);
    else unpack8<kBf16>(q, w);
  }
}

// Weight j of gamma as fp32 (any weight type).
__device__ __forceinline__ float weight_at(const void* __restrict__ gamma, int wdt, int j) {
  if (wdt == kF32) return static_cast<const float*>(gamma)[j];
  const uint32_t b = static_cast<const uint16_t*>(gamma)[j];
  return wdt == kF16 ? f16_pair(b).x : bf16_lo(b);
}

// The 8 weights of group c (columns 8c .. 8c + 7), zero past D, with the
// zero-centred offset: a full group as one vector read, the partial last
// group element by element (so nothing past gamma's D values is read).
__device__ __forceinline__ void weights_group(const void* __restrict__ gamma, int wdt, int zc, int D,
                                              int c, float (&w)[8]) {
  if (8 * c + 8 <= D) {
    weights8(gamma, wdt, c, w);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = 8 * c + e < D ? weight_at(gamma, wdt, 8 * c + e) : 0.0f;
  }
  if (zc) {
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = w[k] + 1.0f;
  }
}

// Rows of any length: this lane's weights for its groups c = v*LPR + l.
template <int LPR, int VPL>
__device__ __forceinline__ void load_weights_any(const void* __restrict__ gamma, int wdt, int zc,
                                                 int D, int l, float (&w)[VPL][8]) {
#pragma unroll
  for (int v = 0; v < VPL; ++v) weights_group(gamma, wdt, zc, D, v * LPR + l, w[v]);
}

// Loads this lane's weights w_eff = fp32(gamma) (+1.0f in fp32 when
// zero-centred) for its vectors c = v*LPR + l; columns past D read as zero.
template <int LPR, int VPL, bool MASKED>
__device__ __forceinline__ void load_weights(const void* __restrict__ gamma, int wdt, int zc,
                                             int nv, int l, float (&w)[VPL][8]) {
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int c = v * LPR + l;
    if (!MASKED || c < nv) {
      weights8(gamma, wdt, c, w[v]);
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
