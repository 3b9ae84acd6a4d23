// Runs every entry point of the CPU oracle (oracle/rmsnorm_oracle.cpp) on
// small seeded inputs in a build with AddressSanitizer and
// UndefinedBehaviorSanitizer: strided rows, batches of 0 and 1 rows, rows of
// 1..130 elements, optional outputs left NULL, and edge values (zeros, +-inf,
// NaN, the largest bf16, subnormals) in every operand. Buffers are sized
// exactly, so a read or write past an operand trips AddressSanitizer. Test
// infrastructure: exit status 0 when every call returns and reports success.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "rmsnorm_oracle.h"

namespace {

int failures = 0;
void ok(int rc, const char* what, long long T, long long D) {
  if (rc != 0) {
    std::fprintf(stderr, "FAIL %s T=%lld D=%lld rc=%d\n", what, T, D, rc);
    ++failures;
  }
}

std::mt19937_64 rng(20261202);

uint16_t bits_of(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return static_cast<uint16_t>(u >> 16);
}

// A [T, ld] bf16 operand: N(0,1) values, plus edge values when `edges`.
std::vector<uint16_t> act(int64_t T, int64_t ld, bool edges) {
  std::normal_distribution<float> n(0.0f, 1.0f);
  std::vector<uint16_t> v(static_cast<size_t>(T * ld));
  const uint16_t special[] = {0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0x7F7F, 0xFF7F, 0x0001, 0x8001};
  for (auto& b : v) b = bits_of(n(rng));
  if (edges)
    for (size_t i = 0; i < v.size(); i += 7) v[i] = special[(i / 7) % 9];
  return v;
}

std::vector<float> vec(int64_t n, float base, float spread) {
  std::normal_distribution<float> d(base, spread);
  std::vector<float> v(static_cast<size_t>(n));
  for (auto& x : v) x = d(rng);
  return v;
}

std::vector<double> dvec(int64_t n) {
  std::normal_distribution<double> d(0.0, 1.0);
  std::vector<double> v(static_cast<size_t>(n));
  for (auto& x : v) x = d(rng);
  return v;
}

// Empty operands (T = 0) still get a valid pointer, as the oracle requires:
// one element of its type, so any access past it trips AddressSanitizer.
template <class V>
auto* ptr(V& v) {
  if (v.empty()) v.resize(1);
  return v.data();
}

void rmsnorm_forms(int64_t T, int64_t D, int64_t pad, bool edges) {
  const int64_t ld = D + pad;
  auto x = act(T, ld, edges), z = act(T, ld, edges), g = act(T, ld, edges), res = act(T, ld, edges);
  auto gamma = vec(D, 1.0f, 0.1f);
  std::vector<uint16_t> y(static_cast<size_t>(T * ld)), r2(static_cast<size_t>(T * ld));
  std::vector<float> rstd(static_cast<size_t>(T)), w(static_cast<size_t>(D)), dg(static_cast<size_t>(D));
  for (int mode : {ORACLE_R64, ORACLE_A32}) {
    for (int zc : {0, 1}) {
      ok(oracle_weights(ptr(gamma), zc, D, ptr(w)), "weights", T, D);
      ok(oracle_rmsnorm_fwd(mode, ptr(x), ld, ptr(gamma), zc, 1e-6f, T, D, ptr(y), ld, ptr(rstd)), "fwd", T, D);
      ok(oracle_rmsnorm_fwd(mode, ptr(x), ld, ptr(gamma), zc, 0.0f, T, D, ptr(y), ld, nullptr), "fwd eps0", T, D);
      ok(oracle_rmsnorm_residual_fwd(mode, ptr(x), ld, ptr(gamma), zc, 1e-6f, T, D, ptr(y), ld, ptr(r2), ld,
                                     ptr(rstd)), "residual_fwd", T, D);
      ok(oracle_rmsnorm_gated_fwd(mode, ptr(x), ld, ptr(z), ld, ptr(gamma), zc, 1e-6f, T, D, ptr(y), ld,
                                  nullptr), "gated_fwd", T, D);
      for (int act_ : {ORACLE_GATE_SILU, ORACLE_GATE_SIGMOID})
        for (int conv : {ORACLE_GATED_FP32, ORACLE_GATED_CAST})
          ok(oracle_rmsnorm_gated_fwd_ex(mode, act_, conv, ptr(x), ld, ptr(z), ld, ptr(gamma), zc, 1e-6f, T,
                                         D, ptr(y), ld, ptr(rstd)), "gated_fwd_ex", T, D);
      ok(oracle_rmsnorm_bwd_dx(mode, ptr(g), ld, ptr(x), ld, ptr(rstd), ptr(gamma), zc, T, D, ptr(res), ld,
                               ptr(y), ld), "bwd_dx gres", T, D);
      ok(oracle_rmsnorm_bwd_dx(mode, ptr(g), ld, ptr(x), ld, ptr(rstd), ptr(gamma), zc, T, D, nullptr, 0,
                               ptr(y), ld), "bwd_dx", T, D);
      ok(oracle_rmsnorm_dgamma(mode, ptr(g), ld, ptr(x), ld, ptr(rstd), T, D, ptr(dg)), "dgamma", T, D);
      for (int act_ : {ORACLE_GATE_SILU, ORACLE_GATE_SIGMOID}) {
        ok(oracle_rmsnorm_gated_bwd(mode, act_, ptr(g), ld, ptr(x), ld, ptr(z), ld, ptr(rstd), ptr(gamma), zc,
                                    T, D, ptr(y), ld, ptr(r2), ld), "gated_bwd", T, D);
        ok(oracle_rmsnorm_gated_bwd(mode, act_, ptr(g), ld, ptr(x), ld, ptr(z), ld, ptr(rstd), ptr(gamma), zc,
                                    T, D, nullptr, 0, ptr(r2), ld), "gated_bwd dz only", T, D);
        ok(oracle_rmsnorm_gated_dgamma(mode, act_, ptr(g), ld, ptr(x), ld, ptr(z), ld, ptr(rstd), T, D,
                                       ptr(dg)), "gated_dgamma", T, D);
      }
      ok(oracle_rmsnorm_add_fwd(mode, ptr(x), ld, ptr(res), ld, ptr(gamma), zc, 1e-6f, T, D, ptr(y), ld,
                                ptr(r2), ld, ptr(rstd)), "add_fwd", T, D);
      ok(oracle_rmsnorm_add_bwd(mode, ptr(g), ld, ptr(x), ld, ptr(res), ld, ptr(rstd), ptr(gamma), zc, T, D,
                                ptr(z), ld, ptr(y), ld, ptr(dg)), "add_bwd", T, D);
      ok(oracle_rmsnorm_add_bwd(mode, ptr(g), ld, ptr(x), ld, ptr(res), ld, ptr(rstd), ptr(gamma), zc, T, D,
                                nullptr, 0, nullptr, 0, ptr(dg)), "add_bwd dgamma only", T, D);
      for (int adt : {ORACLE_BF16, ORACLE_F16})
        for (int wdt : {ORACLE_F32, ORACLE_BF16, ORACLE_F16}) {
          // weights of every type from the same buffer (fp32 holds enough bytes)
          ok(oracle_rmsnorm_fwd_dt(mode, adt, wdt, ptr(x), ld, ptr(gamma), zc, 1e-6f, T, D, ptr(y), ld,
                                   ptr(rstd)), "fwd_dt", T, D);
          ok(oracle_rmsnorm_bwd_dx_dt(mode, adt, wdt, ptr(g), ld, ptr(x), ld, ptr(rstd), ptr(gamma), zc, T, D,
                                      ptr(res), ld, ptr(y), ld), "bwd_dx_dt", T, D);
          ok(oracle_rmsnorm_dgamma_dt(mode, adt, ptr(g), ld, ptr(x), ld, ptr(rstd), T, D, ptr(dg)),
             "dgamma_dt", T, D);
        }
    }
  }
}

void exact_forms(int64_t T, int64_t D) {
  auto x = dvec(T * D), z = dvec(T * D), g = dvec(T * D), res = dvec(T * D), gamma = dvec(D);
  std::vector<double> y(static_cast<size_t>(T * D)), dx(static_cast<size_t>(T * D)),
      dz(static_cast<size_t>(T * D)), h(static_cast<size_t>(T * D)), r(static_cast<size_t>(T)),
      dg(static_cast<size_t>(D));
  for (int zc : {0, 1}) {
    ok(oracle_rmsnorm_fwd_f64(ptr(x), ptr(gamma), zc, 1e-6, T, D, ptr(y), ptr(r)), "fwd_f64", T, D);
    ok(oracle_rmsnorm_gated_fwd_f64(ptr(x), ptr(z), ptr(gamma), zc, 1e-6, T, D, ptr(y)), "gated_fwd_f64", T, D);
    ok(oracle_rmsnorm_bwd_f64(ptr(g), ptr(x), ptr(gamma), zc, 1e-6, T, D, ptr(res), ptr(dx), ptr(dg)),
       "bwd_f64", T, D);
    ok(oracle_rmsnorm_bwd_f64(ptr(g), ptr(x), ptr(gamma), zc, 1e-6, T, D, nullptr, nullptr, ptr(dg)),
       "bwd_f64 dgamma only", T, D);
    for (int act_ : {ORACLE_GATE_SILU, ORACLE_GATE_SIGMOID}) {
      ok(oracle_rmsnorm_gated_fwd_ex_f64(act_, ptr(x), ptr(z), ptr(gamma), zc, 1e-6, T, D, ptr(y)),
         "gated_fwd_ex_f64", T, D);
      ok(oracle_rmsnorm_gated_bwd_f64(act_, ptr(g), ptr(x), ptr(z), ptr(gamma), zc, 1e-6, T, D, ptr(dx),
                                      ptr(dz), ptr(dg)), "gated_bwd_f64", T, D);
    }
    ok(oracle_rmsnorm_add_fwd_f64(ptr(x), ptr(res), ptr(gamma), zc, 1e-6, T, D, ptr(y), ptr(h), ptr(r)),
       "add_fwd_f64", T, D);
    ok(oracle_rmsnorm_add_bwd_f64(ptr(g), ptr(x), ptr(res), ptr(gamma), zc, 1e-6, T, D, ptr(z), ptr(dx),
                                  ptr(dg)), "add_bwd_f64", T, D);
  }
  // the fp32-input gated forward
  std::vector<float> xf(static_cast<size_t>(T * D)), zf(xf.size()), of(xf.size());
  auto gf = vec(D, 1.0f, 0.1f);
  for (size_t i = 0; i < xf.size(); ++i) { xf[i] = static_cast<float>(x[i]); zf[i] = static_cast<float>(z[i]); }
  ok(oracle_rmsnorm_gated_fwd_f32io(ORACLE_GATE_SILU, ORACLE_GATED_CAST, ptr(xf), ptr(zf), ptr(gf), 1, 1e-6f,
                                    T, D, ptr(of)), "gated_fwd_f32io", T, D);
}

void codecs_and_gemm() {
  std::vector<uint16_t> b(1 << 16);
  for (size_t i = 0; i < b.size(); ++i) b[i] = static_cast<uint16_t>(i);
  std::vector<float> f(b.size());
  oracle_bf16_decode(b.data(), static_cast<int64_t>(b.size()), f.data());
  oracle_bf16_encode(f.data(), static_cast<int64_t>(f.size()), b.data());
  oracle_f16_decode(b.data(), static_cast<int64_t>(b.size()), f.data());
  oracle_f16_encode(f.data(), static_cast<int64_t>(f.size()), b.data());
  for (int64_t M : {0, 1, 5})
    for (int64_t N : {0, 1, 3})
      for (int64_t K : {32, 64}) {
        const int64_t ldx = K + 8, ldw = K + 16, ldy = N + 3;
        auto X = act(M, ldx, true), W = act(N, ldw, true);
        std::vector<uint16_t> Y(static_cast<size_t>(M * ldy));
        std::vector<double> E(static_cast<size_t>(M * N));
        ok(oracle_gemm_xwt(ptr(X), ldx, ptr(W), ldw, M, N, K, ptr(Y), ldy, ptr(E)), "gemm", M, N);
        ok(oracle_gemm_xwt(ptr(X), ldx, ptr(W), ldw, M, N, K, ptr(Y), ldy, nullptr), "gemm no exact", M, N);
      }
}

}  // namespace

int main() {
  for (int64_t T : {0, 1, 3, 17})
    for (int64_t D : {1, 2, 7, 8, 13, 64, 100, 130})
      for (int64_t pad : {0, 3})
        for (bool edges : {false, true}) rmsnorm_forms(T, D, pad, edges);
  for (int m : {1, 2, 0}) {
    oracle_set_mutation(m);
    rmsnorm_forms(5, 24, 1, false);
    exact_forms(3, 16);
  }
  for (int64_t T : {0, 1, 2, 3})
    for (int64_t D : {1, 8, 16, 37}) exact_forms(T, D);
  codecs_and_gemm();
  std::printf("oracle sanitizer cases: %d failures\n", failures);
  return failures == 0 ? 0 : 1;
}
