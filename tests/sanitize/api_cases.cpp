// Drives every C entry point of api.cpp, linked with launch_stub.cpp, over
// ordinary and extreme arguments (sizes near INT64_MAX, negative strides,
// strides at and past the limits, misaligned and overlapping fake pointers)
// in a build with AddressSanitizer and UndefinedBehaviorSanitizer: the host
// validation must return a valid status for every call without undefined
// behaviour (no signed overflow in its size arithmetic), launch only what it
// accepts, and accept ordinary calls. Fake device addresses are never
// dereferenced. Exit status 0 on success.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "rmsnorm_mi355x.h"

extern int g_launches;

namespace {

int failures = 0;
void expect(bool ok, const char* what, long long a = 0, long long b = 0, long long c = 0) {
  if (!ok) {
    std::fprintf(stderr, "FAIL %s (%lld, %lld, %lld)\n", what, a, b, c);
    ++failures;
  }
}

bool valid_status(int s) { return s >= RMSN_OK && s <= RMSN_ERR_MODE; }

template <class T> T* P(uintptr_t a) { return reinterpret_cast<T*>(a); }
constexpr uintptr_t kA = 0x7F0000000000, kStep = uintptr_t{1} << 36;
uint16_t* act(int i) { return P<uint16_t>(kA + i * kStep); }
float* f32(int i) { return P<float>(kA + i * kStep); }

const int64_t kBig = INT64_MAX;
const std::vector<int64_t> kT = {-1, 0, 1, 7, 1000, int64_t{1} << 31, int64_t{1} << 40,
                                 int64_t{1} << 62, kBig - 1, kBig};
const std::vector<int64_t> kD = {-1, 0, 1, 7, 8, 100, 4096, 32767, 32768, 32769,
                                 int64_t{1} << 40, kBig};
const std::vector<int64_t> kLdDelta = {-1, 0, 1, 8, (int64_t{1} << 24), kBig};

// ld values derived from D: D + delta (saturating), plus absolute extremes
std::vector<int64_t> lds(int64_t D) {
  std::vector<int64_t> v = {-5, 0, int64_t{1} << 24, (int64_t{1} << 24) + 8, kBig};
  for (int64_t d : kLdDelta) {
    const __int128 w = static_cast<__int128>(D) + d;  // saturated to int64
    v.push_back(w > kBig ? kBig : w < INT64_MIN ? INT64_MIN : static_cast<int64_t>(w));
  }
  return v;
}

void sweep_forward() {
  for (int64_t T : kT)
    for (int64_t D : kD)
      for (int64_t ld : lds(D)) {
        const int before = g_launches;
        int s = rmsnorm_fwd(act(0), ld, f32(5), 0, 1e-6f, T, D, act(1), ld, f32(6), nullptr);
        expect(valid_status(s), "fwd status", T, D, ld);
        expect(s == RMSN_OK || g_launches == before, "fwd launched on error", T, D, ld);
        s = rmsnorm_residual_fwd(act(0), ld, f32(5), 1, 0.0f, T, D, act(1), ld, act(2), ld,
                                 nullptr, nullptr);
        expect(valid_status(s), "residual status", T, D, ld);
        s = rmsnorm_gated_fwd_ex(act(0), ld, act(3), ld, f32(5), 0, 1e-6f, T, D, 1, 1, act(1), ld,
                                 f32(6), nullptr);
        expect(valid_status(s), "gated status", T, D, ld);
        s = rmsnorm_add_fwd(act(0), ld, act(3), ld, f32(5), 0, 1e-6f, T, D, act(0), ld, act(3), ld,
                            f32(6), nullptr);
        expect(valid_status(s), "add status", T, D, ld);
        s = rmsnorm_fwd_dt(RMSN_DTYPE_F16, RMSN_DTYPE_BF16, act(0), ld, f32(5), 0, 1e-6f, T, D,
                           act(1), ld, nullptr, nullptr);
        expect(valid_status(s), "fwd_dt status", T, D, ld);
      }
}

void sweep_backward() {
  const std::vector<size_t> ws_bytes = {0, 16, size_t{1} << 30, SIZE_MAX};
  for (int64_t T : kT)
    for (int64_t D : kD) {
      const size_t need = rmsnorm_bwd_workspace_bytes(T, D);
      int64_t R = -1, S = -1, K = -1;
      const int ls = rmsnorm_bwd_partials_layout(T, D, &R, &S, &K);
      expect(valid_status(ls), "layout status", T, D);
      if (ls == RMSN_OK) {
        expect(R >= 1 && S >= 1 && K >= 0 && K <= 512, "layout values", R, S, K);
        expect(need == (T > 0 ? size_t(K) * size_t((D + 7) / 8 * 8) * 4 : 0), "workspace bytes", T, D);
        expect(rmsnorm_dgamma_chunk_rows(D) == R, "chunk rows", D, R);
      }
      for (int64_t ld : lds(D))
        for (size_t wb : ws_bytes) {
          const int before = g_launches;
          int s = rmsnorm_bwd(act(0), ld, act(1), ld, f32(6), f32(5), 0, T, D, act(3), ld, act(2),
                              ld, f32(7), f32(8), wb, nullptr);
          expect(valid_status(s), "bwd status", T, D, ld);
          expect(s == RMSN_OK || g_launches == before, "bwd launched on error", T, D, ld);
          s = rmsnorm_bwd_rows(act(0), ld, act(1), ld, f32(6), f32(5), 1, T, D, nullptr, 0, act(2),
                               ld, f32(8), wb, nullptr);
          expect(valid_status(s), "bwd_rows status", T, D, ld);
          s = rmsnorm_bwd_finish(f32(8), wb, T, D, f32(7), nullptr);
          expect(valid_status(s), "finish status", T, D, ld);
          s = rmsnorm_gated_bwd(act(0), ld, act(1), ld, act(3), ld, f32(6), f32(5), 0, T, D, 0,
                                act(2), ld, act(4), ld, f32(7), f32(8), wb, nullptr);
          expect(valid_status(s), "gated_bwd status", T, D, ld);
          s = rmsnorm_add_bwd(act(0), ld, act(1), ld, act(3), ld, f32(6), f32(5), 0, T, D, act(4),
                              ld, act(2), ld, f32(7), f32(8), wb, nullptr);
          expect(valid_status(s), "add_bwd status", T, D, ld);
          s = rmsnorm_bwd_dt(RMSN_DTYPE_F16, RMSN_DTYPE_F16, act(0), ld, act(1), ld, f32(6), f32(5),
                             1, T, D, nullptr, 0, act(2), ld, f32(7), f32(8), wb, nullptr);
          expect(valid_status(s), "bwd_dt status", T, D, ld);
        }
      const int s = rmsnorm_bwd_noalloc(act(0), D, act(1), D, f32(6), f32(5), 0, T, D, nullptr, 0,
                                        act(2), D, f32(7), nullptr);
      expect(valid_status(s), "noalloc status", T, D);
    }
}

void sweep_gemm() {
  const std::vector<int64_t> sizes = {-1, 0, 1, 32, 4096, int64_t{1} << 31, int64_t{1} << 40, kBig};
  for (int64_t M : sizes)
    for (int64_t N : sizes)
      for (int64_t K : sizes)
        for (int64_t ld : {int64_t{4096}, int64_t{1} << 21, (int64_t{1} << 21) + 8, kBig, int64_t{-8}}) {
          const int before = g_launches;
          const int s = bigemm_bf16_xwt(act(0), ld, act(1), ld, M, N, K, act(2), ld, nullptr);
          expect(valid_status(s), "gemm status", M, N, K);
          expect(s == RMSN_OK || g_launches == before, "gemm launched on error", M, N, K);
          int64_t tm = 0, tn = 0;
          expect(valid_status(bigemm_bf16_tile(M, N, &tm, &tn)), "tile status", M, N);
        }
}

void known_answers() {
  // ordinary calls are accepted and launch; a few rejections keep their codes
  int before = g_launches;
  expect(rmsnorm_fwd(act(0), 4096, f32(5), 0, 1e-6f, 32768, 4096, act(1), 4096, f32(6), nullptr) ==
             RMSN_OK && g_launches == before + 1, "fwd accepted");
  before = g_launches;
  expect(rmsnorm_bwd(act(0), 4096, act(1), 4096, f32(6), f32(5), 0, 32768, 4096, nullptr, 0,
                     act(2), 4096, f32(7), f32(8), size_t{1} << 30, nullptr) == RMSN_OK &&
             g_launches == before + 2, "bwd accepted");
  before = g_launches;
  expect(rmsnorm_bwd_noalloc(act(0), 4100, act(1), 4100, f32(6), f32(5), 1, 999, 4100, act(3), 4100,
                             act(2), 4100, f32(7), nullptr) == RMSN_OK &&
             g_launches == before + 2, "noalloc accepted");
  before = g_launches;
  expect(bigemm_bf16_xwt(act(0), 4096, act(1), 4096, 4096, 4096, 4096, act(2), 4096, nullptr) ==
             RMSN_OK && g_launches == before + 1, "gemm accepted");
  expect(rmsnorm_fwd(act(0), 4096, f32(5), 0, 1e-6f, 8, 4096, act(0), 4096, nullptr, nullptr) ==
             RMSN_ERR_ALIASING, "fwd in place rejected");
  expect(rmsnorm_bwd(act(0), 4096, act(1), 4096, f32(6), f32(5), 0, 1000, 4096, nullptr, 0, act(2),
                     4096, f32(7), f32(8), 16, nullptr) == RMSN_ERR_WORKSPACE, "small workspace");
  expect(bigemm_bf16_xwt(act(0), 4096, act(1), 4096, 64, 4096, 4096, act(2), int64_t{1} << 61,
                         nullptr) == RMSN_ERR_SHAPE, "gemm ld_y bound");
}

}  // namespace

int main() {
  known_answers();
  sweep_forward();
  sweep_backward();
  sweep_gemm();
  std::printf("api sanitizer cases: %d failures, %d launches accepted\n", failures, g_launches);
  return failures == 0 ? 0 : 1;
}
