// Host-only stand-ins for the kernel launchers, linked with api.cpp in the
// sanitizer build (tests/test_sanitizers.py): no GPU, nothing launched. Each
// stub checks the invariants the real launcher and its kernels rely on
// (what api.cpp promises to pass after its checks) and counts the calls.
#include <cstdio>
#include <cstdlib>

#include "geometry.hpp"
#include "launch.hpp"
#include "scratch.hpp"

namespace {
[[noreturn]] void fail(const char* what) {
  std::fprintf(stderr, "launch contract broken: %s\n", what);
  std::abort();
}
void require(bool ok, const char* what) {
  if (!ok) fail(what);
}
}  // namespace

int g_launches = 0;

namespace rmsn {

int launch_fwd(const FwdArgs& a, void*) {
  require(a.T > 0 && a.D >= 1 && a.D <= 32768, "fwd sizes");
  require(a.x != nullptr && a.y != nullptr && a.gamma != nullptr, "fwd pointers");
  require(a.ld_x >= a.D && a.ld_y >= a.D && a.ld_x <= (1 << 24) && a.ld_y <= (1 << 24), "fwd strides");
  require(a.res == nullptr || (a.ld_res >= a.D && a.ld_res <= (1 << 24)), "fwd residual stride");
  require(a.z == nullptr || (a.ld_z >= a.D && a.ld_z <= (1 << 24)), "fwd gate stride");
  require(a.rin == nullptr || (a.ld_rin >= a.D && a.ld_rin <= (1 << 24)), "fwd add stride");
  ++g_launches;
  return 0;
}

int launch_bwd_rows(const BwdArgs& a, void*) {
  require(a.T > 0 && a.D >= 1 && a.D <= 32768, "bwd sizes");
  require(a.g != nullptr && a.x != nullptr && a.rstd != nullptr && a.gamma != nullptr, "bwd pointers");
  require(a.dx != nullptr || a.part != nullptr, "bwd writes something");
  require(a.chunks >= 1 && a.chunks <= kMaxChunks && a.group_blocks >= 1, "bwd chunking");
  require(a.ld_g >= a.D && a.ld_x >= a.D && a.ld_g <= (1 << 24) && a.ld_x <= (1 << 24), "bwd strides");
  require(a.dx == nullptr || (a.ld_dx >= a.D && a.ld_dx <= (1 << 24)), "bwd dx stride");
  ++g_launches;
  return 0;
}

int launch_bwd_finish(const float* part, int64_t chunks, int D, float* dgamma, void*) {
  require(chunks >= 0 && chunks <= kMaxChunks && D >= 1 && D <= 32768, "finish sizes");
  require(dgamma != nullptr && (chunks == 0 || part != nullptr), "finish pointers");
  ++g_launches;
  return 0;
}

int launch_gemm(const GemmArgs& a, void*) {
  require(a.M > 0 && a.N > 0 && a.K > 0 && a.K % 32 == 0, "gemm sizes");
  require(a.ld_x >= a.K && a.ld_w >= a.K && a.ld_y >= a.N, "gemm strides");
  require(a.x != nullptr && a.w != nullptr && a.y != nullptr, "gemm pointers");
  ++g_launches;
  return 0;
}

void gemm_tile(int64_t M, int64_t N, int64_t* bm, int64_t* bn) {
  require(M >= 0 && N >= 0, "gemm tile sizes");
  *bm = 32;
  *bn = 64;
}

int scratch_ptr(void** out) {
  // a fake, aligned device address: the stubs never dereference it
  *out = reinterpret_cast<void*>(uintptr_t{0x7E0000000000});
  return 0;
}

}  // namespace rmsn
