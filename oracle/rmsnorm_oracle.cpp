// CPU oracle for batch-invariant RMSNorm — TEST INFRASTRUCTURE ONLY.
// Only the tests, the smoke check and the benchmark's CPU-baseline leg may
// load it. Build: g++ -std=c++17 -O2 -ffp-contract=off (no fast-math), so
// every `float` expression below is exactly one IEEE fp32 operation rounded
// to nearest-even. Sources and modes are described in rmsnorm_oracle.h.
#include "rmsnorm_oracle.h"

#include <cmath>
#include <cstring>

namespace {

int g_mutation = 0;

float bf16_to_f32(uint16_t b) {
  uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Round to nearest, ties to even: add 0x7FFF plus the lowest kept bit, then
// drop the low 16 bits. A carry out of the mantissa moves into the exponent,
// which is also how values past the largest bf16 become infinity.
uint16_t f32_to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u)  // NaN: keep sign, force quiet bit
    return static_cast<uint16_t>((u >> 16) | 0x0040u);
  const uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return static_cast<uint16_t>(u >> 16);
}

bool bad_2d(const void* p, int64_t ld, int64_t D) { return p == nullptr || ld < D; }

// w_eff = fp32(gamma) (+ 1.0f in fp32 when zero-centred).
float weight_eff(const float* gamma, int zc, int64_t j) {
  float w = gamma[j];
  if (zc) w = w + 1.0f;
  return w;
}

// A reduction of fp32 terms in ascending order: in double, rounded once (R64)
// or in fp32 (A32).
struct Sum {
  int mode;
  double d = 0.0;
  float f = 0.0f;
  explicit Sum(int m) : mode(m) {}
  void add(float t) {
    if (mode == ORACLE_A32)
      f = f + t;
    else
      d = d + static_cast<double>(t);
  }
  float value() const { return mode == ORACLE_A32 ? f : static_cast<float>(d); }
};

// rsqrt(v) = 1/sqrt(v) in double, rounded to fp32.
float rsqrt_ref(float v) {
  return static_cast<float>(1.0 / std::sqrt(static_cast<double>(v)));
}

// Steps (i)-(v) of the forward for one row: the row's rstd.
float row_rstd(int mode, const uint16_t* xr, int64_t D, float eps) {
  Sum ss(mode);
  for (int64_t j = 0; j < D; ++j) {
    const float xf = bf16_to_f32(xr[j]);
    const float sq = xf * xf;
    ss.add(sq);
  }
  const float mean = ss.value() / static_cast<float>(D);
  const float v = mean + eps;
  return rsqrt_ref(v);
}

// n_j = (x_j * r) * w_j, the normalised and weighted value before rounding.
float row_normed(float xf, float r, float w) {
  const float xr = xf * r;
  return xr * w;
}

bool bad_mode(int mode) { return mode != ORACLE_R64 && mode != ORACLE_A32; }

double silu_d(double z) { return z / (1.0 + std::exp(-z)); }

double sigmoid_d(double z) { return 1.0 / (1.0 + std::exp(-z)); }

// sigmoid(z) and 1 - sigmoid(z) in double, both from e = exp(-|z|):
// 1/(1+e) and e/(1+e), assigned by the sign of z. Neither comes from a
// subtraction 1 - s, which would lose the relative precision of the small
// one (for z = 30, 1 - s is about 1e-13).
void sigmoid_pair_d(double z, double& s, double& sc) {
  const double e = std::exp(-std::fabs(z));
  const double inv = 1.0 / (1.0 + e);
  s = z >= 0.0 ? inv : e * inv;
  sc = z >= 0.0 ? e * inv : inv;
}

// The gate a(z) and its derivative, in double: silu' = s (1 + z (1 - s)),
// sigmoid' = s (1 - s).
double gate_d(int act, double z) { return act == ORACLE_GATE_SIGMOID ? sigmoid_d(z) : silu_d(z); }
double gate_grad_d(int act, double z) {
  double s, sc;
  sigmoid_pair_d(z, s, sc);
  return act == ORACLE_GATE_SIGMOID ? s * sc : s * (1.0 + z * sc);
}
bool bad_act(int act) { return act != ORACLE_GATE_SILU && act != ORACLE_GATE_SIGMOID; }

// bf16 rounding of an fp32 value, returned as fp32 (the cast to the input
// dtype in the cast convention).
float round_bf16(float v) { return bf16_to_f32(f32_to_bf16(v)); }

}  // namespace

extern "C" {

void oracle_set_mutation(int mutation) { g_mutation = mutation; }

void oracle_bf16_decode(const uint16_t* in, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_to_f32(in[i]);
}

void oracle_bf16_encode(const float* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16(in[i]);
}

int oracle_weights(const float* gamma, int zero_centered, int64_t D, float* w_eff) {
  if (!gamma || !w_eff || D <= 0) return -1;
  for (int64_t j = 0; j < D; ++j) w_eff[j] = weight_eff(gamma, zero_centered, j);
  return 0;
}

static int fwd_common(int mode, const uint16_t* x, int64_t ld_x, const uint16_t* z,
                      int64_t ld_z, const float* gamma, int zc, float eps, int64_t T,
                      int64_t D, uint16_t* y, int64_t ld_y, uint16_t* res,
                      int64_t ld_res, float* rstd) {
  if (bad_mode(mode) || T < 0 || D <= 0 || !gamma || bad_2d(x, ld_x, D) ||
      bad_2d(y, ld_y, D))
    return -1;
  // Defect 1 of [MEG] (test-only): the forward reads the raw weight.
  const int zc_fwd = (g_mutation == 1) ? 0 : zc;
  for (int64_t t = 0; t < T; ++t) {
    const uint16_t* xr = x + t * ld_x;
    const float r = row_rstd(mode, xr, D, eps);
    if (rstd) rstd[t] = r;
    for (int64_t j = 0; j < D; ++j) {
      const float n = row_normed(bf16_to_f32(xr[j]), r, weight_eff(gamma, zc_fwd, j));
      float o = n;
      if (z) {
        const float zf = bf16_to_f32(z[t * ld_z + j]);
        const float sg = static_cast<float>(silu_d(static_cast<double>(zf)));
        o = n * sg;
      }
      y[t * ld_y + j] = f32_to_bf16(o);
      if (res) res[t * ld_res + j] = xr[j];
    }
  }
  return 0;
}

int oracle_rmsnorm_fwd(int mode, const uint16_t* x, int64_t ld_x, const float* gamma,
                       int zero_centered, float eps, int64_t T, int64_t D, uint16_t* y,
                       int64_t ld_y, float* rstd) {
  return fwd_common(mode, x, ld_x, nullptr, 0, gamma, zero_centered, eps, T, D, y, ld_y,
                    nullptr, 0, rstd);
}

int oracle_rmsnorm_residual_fwd(int mode, const uint16_t* x, int64_t ld_x,
                                const float* gamma, int zero_centered, float eps,
                                int64_t T, int64_t D, uint16_t* y, int64_t ld_y,
                                uint16_t* residual_out, int64_t ld_res, float* rstd) {
  if (bad_2d(residual_out, ld_res, D)) return -1;
  return fwd_common(mode, x, ld_x, nullptr, 0, gamma, zero_centered, eps, T, D, y, ld_y,
                    residual_out, ld_res, rstd);
}

int oracle_rmsnorm_gated_fwd(int mode, const uint16_t* x, int64_t ld_x, const uint16_t* z,
                             int64_t ld_z, const float* gamma, int zero_centered, float eps,
                             int64_t T, int64_t D, uint16_t* out, int64_t ld_out,
                             float* rstd) {
  if (bad_2d(z, ld_z, D)) return -1;
  return fwd_common(mode, x, ld_x, z, ld_z, gamma, zero_centered, eps, T, D, out, ld_out,
                    nullptr, 0, rstd);
}

int oracle_rmsnorm_bwd_dx(int mode, const uint16_t* g, int64_t ld_g, const uint16_t* x,
                          int64_t ld_x, const float* rstd, const float* gamma,
                          int zero_centered, int64_t T, int64_t D, const uint16_t* gres,
                          int64_t ld_gres, uint16_t* dx, int64_t ld_dx) {
  if (bad_mode(mode) || T < 0 || D <= 0 || !gamma || !rstd || bad_2d(g, ld_g, D) ||
      bad_2d(x, ld_x, D) || bad_2d(dx, ld_dx, D) || (gres && ld_gres < D))
    return -1;
  for (int64_t t = 0; t < T; ++t) {
    const uint16_t* gr = g + t * ld_g;
    const uint16_t* xr = x + t * ld_x;
    const float r = rstd[t];
    Sum s(mode);
    for (int64_t i = 0; i < D; ++i) {
      const float gw = bf16_to_f32(gr[i]) * weight_eff(gamma, zero_centered, i);
      const float term = gw * bf16_to_f32(xr[i]);
      s.add(term);
    }
    const float r2 = r * r;
    const float r3 = r2 * r;
    const float r3s = r3 * s.value();
    const float c = r3s / static_cast<float>(D);
    for (int64_t k = 0; k < D; ++k) {
      const float w = weight_eff(gamma, zero_centered, k);
      const float xf = bf16_to_f32(xr[k]);
      const float gw = bf16_to_f32(gr[k]) * w;
      const float t1 = gw * r;
      float t2 = xf * c;
      if (g_mutation == 2) t2 = t2 * w;  // defect 2 of [MEG] (test-only)
      float d = t1 - t2;
      if (gres) d = d + bf16_to_f32(gres[t * ld_gres + k]);
      dx[t * ld_dx + k] = f32_to_bf16(d);
    }
  }
  return 0;
}

int oracle_rmsnorm_dgamma(int mode, const uint16_t* g, int64_t ld_g, const uint16_t* x,
                          int64_t ld_x, const float* rstd, int64_t T, int64_t ncols,
                          float* dgamma) {
  if (bad_mode(mode) || T < 0 || ncols <= 0 || !dgamma || bad_2d(g, ld_g, ncols) ||
      bad_2d(x, ld_x, ncols) || (T > 0 && !rstd))
    return -1;
  for (int64_t j = 0; j < ncols; ++j) {
    Sum acc(mode);
    for (int64_t t = 0; t < T; ++t) {
      const float gx = bf16_to_f32(g[t * ld_g + j]) * bf16_to_f32(x[t * ld_x + j]);
      const float term = gx * rstd[t];
      acc.add(term);
    }
    dgamma[j] = acc.value();
  }
  return 0;
}

// ---- gated-norm variants -----------------------------------------------------

int oracle_rmsnorm_gated_fwd_ex(int mode, int activation, int convention, const uint16_t* x,
                                int64_t ld_x, const uint16_t* z, int64_t ld_z, const float* gamma,
                                int zero_centered, float eps, int64_t T, int64_t D, uint16_t* out,
                                int64_t ld_out, float* rstd) {
  if (bad_mode(mode) || bad_act(activation) ||
      (convention != ORACLE_GATED_FP32 && convention != ORACLE_GATED_CAST) || T < 0 || D <= 0 ||
      !gamma || bad_2d(x, ld_x, D) || bad_2d(z, ld_z, D) || bad_2d(out, ld_out, D))
    return -1;
  const int zc_fwd = (g_mutation == 1) ? 0 : zero_centered;
  for (int64_t t = 0; t < T; ++t) {
    const uint16_t* xr = x + t * ld_x;
    const float r = row_rstd(mode, xr, D, eps);
    if (rstd) rstd[t] = r;
    for (int64_t j = 0; j < D; ++j) {
      const float w = weight_eff(gamma, zc_fwd, j);
      const float a = static_cast<float>(gate_d(activation, bf16_to_f32(z[t * ld_z + j])));
      float n = bf16_to_f32(xr[j]) * r;
      if (convention == ORACLE_GATED_CAST) n = round_bf16(n);
      float nw = n * w;
      if (convention == ORACLE_GATED_CAST) nw = round_bf16(nw);
      const float o = nw * a;
      out[t * ld_out + j] = f32_to_bf16(o);
    }
  }
  return 0;
}

int oracle_rmsnorm_gated_fwd_f32io(int activation, int convention, const float* x, const float* z,
                                   const float* gamma, int zero_centered, float eps, int64_t T,
                                   int64_t D, float* out) {
  if (bad_act(activation) || (convention != ORACLE_GATED_FP32 && convention != ORACLE_GATED_CAST) ||
      !x || !z || !gamma || !out || T < 0 || D <= 0)
    return -1;
  for (int64_t t = 0; t < T; ++t) {
    const float* xr = x + t * D;
    double ss = 0.0;
    for (int64_t j = 0; j < D; ++j) {
      const float sq = xr[j] * xr[j];
      ss += static_cast<double>(sq);
    }
    const float mean = static_cast<float>(ss) / static_cast<float>(D);
    const float r = rsqrt_ref(mean + eps);
    for (int64_t j = 0; j < D; ++j) {
      const float w = weight_eff(gamma, zero_centered, j);
      const float a = static_cast<float>(gate_d(activation, static_cast<double>(z[t * D + j])));
      // the casts to the input dtype are the identity for fp32 inputs
      const float n = xr[j] * r;
      const float nw = n * w;
      out[t * D + j] = nw * a;
    }
  }
  return 0;
}

int oracle_rmsnorm_gated_bwd(int mode, int activation, const uint16_t* g, int64_t ld_g,
                             const uint16_t* x, int64_t ld_x, const uint16_t* z, int64_t ld_z,
                             const float* rstd, const float* gamma, int zero_centered, int64_t T,
                             int64_t D, uint16_t* dx, int64_t ld_dx, uint16_t* dz, int64_t ld_dz) {
  if (bad_mode(mode) || bad_act(activation) || T < 0 || D <= 0 || !gamma || !rstd ||
      bad_2d(g, ld_g, D) || bad_2d(x, ld_x, D) || bad_2d(z, ld_z, D) || (!dx && !dz) ||
      (dx && ld_dx < D) || (dz && ld_dz < D))
    return -1;
  for (int64_t t = 0; t < T; ++t) {
    const uint16_t* gr = g + t * ld_g;
    const uint16_t* xr = x + t * ld_x;
    const uint16_t* zr = z + t * ld_z;
    const float r = rstd[t];
    Sum s(mode);
    for (int64_t i = 0; i < D; ++i) {
      const float a = static_cast<float>(gate_d(activation, bf16_to_f32(zr[i])));
      const float gn = bf16_to_f32(gr[i]) * a;
      const float gw = gn * weight_eff(gamma, zero_centered, i);
      const float term = gw * bf16_to_f32(xr[i]);
      s.add(term);
    }
    const float r2 = r * r;
    const float r3 = r2 * r;
    const float r3s = r3 * s.value();
    const float c = r3s / static_cast<float>(D);
    for (int64_t k = 0; k < D; ++k) {
      const float w = weight_eff(gamma, zero_centered, k);
      const float xf = bf16_to_f32(xr[k]);
      const float gf = bf16_to_f32(gr[k]);
      const double zd = bf16_to_f32(zr[k]);
      const float a = static_cast<float>(gate_d(activation, zd));
      const float da = static_cast<float>(gate_grad_d(activation, zd));
      if (dz) {
        const float n = xf * r;
        const float nw = n * w;
        const float gnw = gf * nw;
        dz[t * ld_dz + k] = f32_to_bf16(gnw * da);
      }
      if (dx) {
        const float gn = gf * a;
        const float gw = gn * w;
        const float t1 = gw * r;
        const float t2 = xf * c;
        dx[t * ld_dx + k] = f32_to_bf16(t1 - t2);
      }
    }
  }
  return 0;
}

int oracle_rmsnorm_gated_dgamma(int mode, int activation, const uint16_t* g, int64_t ld_g,
                                const uint16_t* x, int64_t ld_x, const uint16_t* z, int64_t ld_z,
                                const float* rstd, int64_t T, int64_t ncols, float* dgamma) {
  if (bad_mode(mode) || bad_act(activation) || T < 0 || ncols <= 0 || !dgamma ||
      bad_2d(g, ld_g, ncols) || bad_2d(x, ld_x, ncols) || bad_2d(z, ld_z, ncols) ||
      (T > 0 && !rstd))
    return -1;
  for (int64_t j = 0; j < ncols; ++j) {
    Sum acc(mode);
    for (int64_t t = 0; t < T; ++t) {
      const float a = static_cast<float>(gate_d(activation, bf16_to_f32(z[t * ld_z + j])));
      const float gn = bf16_to_f32(g[t * ld_g + j]) * a;
      const float gx = gn * bf16_to_f32(x[t * ld_x + j]);
      const float term = gx * rstd[t];
      acc.add(term);
    }
    dgamma[j] = acc.value();
  }
  return 0;
}

// ---- fused add-RMSNorm ------------------------------------------------------
// The decoder-norm residual path of [C1] ("fused_add_rms_norm, which
// normalises the fp32 sum"): h = fp32(x) + fp32(residual), rounded once to
// fp32; the norm of h; the updated residual stored as bf16(h).

// One row of h = x + residual in fp32.
static void row_sum_inputs(const uint16_t* xr, const uint16_t* rr, int64_t D, float* h) {
  for (int64_t j = 0; j < D; ++j) h[j] = bf16_to_f32(xr[j]) + bf16_to_f32(rr[j]);
}

// rstd of an fp32 row: ss = ascending sum of the fp32 squares fp32(h*h).
static float row_rstd_f32(int mode, const float* h, int64_t D, float eps) {
  Sum ss(mode);
  for (int64_t j = 0; j < D; ++j) {
    const float sq = h[j] * h[j];
    ss.add(sq);
  }
  const float mean = ss.value() / static_cast<float>(D);
  const float v = mean + eps;
  return rsqrt_ref(v);
}

int oracle_rmsnorm_add_fwd(int mode, const uint16_t* x, int64_t ld_x, const uint16_t* residual,
                           int64_t ld_res, const float* gamma, int zero_centered, float eps,
                           int64_t T, int64_t D, uint16_t* y, int64_t ld_y,
                           uint16_t* residual_out, int64_t ld_rout, float* rstd) {
  if (bad_mode(mode) || T < 0 || D <= 0 || !gamma || bad_2d(x, ld_x, D) ||
      bad_2d(residual, ld_res, D) || bad_2d(y, ld_y, D) || bad_2d(residual_out, ld_rout, D))
    return -1;
  float* h = new float[static_cast<size_t>(D)];
  for (int64_t t = 0; t < T; ++t) {
    row_sum_inputs(x + t * ld_x, residual + t * ld_res, D, h);
    const float r = row_rstd_f32(mode, h, D, eps);
    if (rstd) rstd[t] = r;
    for (int64_t j = 0; j < D; ++j) {
      const float n = row_normed(h[j], r, weight_eff(gamma, zero_centered, j));
      y[t * ld_y + j] = f32_to_bf16(n);
      residual_out[t * ld_rout + j] = f32_to_bf16(h[j]);
    }
  }
  delete[] h;
  return 0;
}

int oracle_rmsnorm_add_bwd(int mode, const uint16_t* g, int64_t ld_g, const uint16_t* x,
                           int64_t ld_x, const uint16_t* residual, int64_t ld_res,
                           const float* rstd, const float* gamma, int zero_centered, int64_t T,
                           int64_t D, const uint16_t* g_rout, int64_t ld_gro, uint16_t* dh,
                           int64_t ld_dh, float* dgamma) {
  if (bad_mode(mode) || T < 0 || D <= 0 || !gamma || (T > 0 && !rstd) || bad_2d(g, ld_g, D) ||
      bad_2d(x, ld_x, D) || bad_2d(residual, ld_res, D) || (!dh && !dgamma) ||
      (dh && ld_dh < D) || (g_rout && ld_gro < D))
    return -1;
  float* h = new float[static_cast<size_t>(D)];
  if (dh) {
    for (int64_t t = 0; t < T; ++t) {
      const uint16_t* gr = g + t * ld_g;
      row_sum_inputs(x + t * ld_x, residual + t * ld_res, D, h);
      const float r = rstd[t];
      Sum s(mode);
      for (int64_t i = 0; i < D; ++i) {
        const float gw = bf16_to_f32(gr[i]) * weight_eff(gamma, zero_centered, i);
        const float term = gw * h[i];
        s.add(term);
      }
      const float r2 = r * r;
      const float r3 = r2 * r;
      const float r3s = r3 * s.value();
      const float c = r3s / static_cast<float>(D);
      for (int64_t k = 0; k < D; ++k) {
        const float gw = bf16_to_f32(gr[k]) * weight_eff(gamma, zero_centered, k);
        const float t1 = gw * r;
        const float t2 = h[k] * c;
        float d = t1 - t2;
        if (g_rout) d = d + bf16_to_f32(g_rout[t * ld_gro + k]);
        dh[t * ld_dh + k] = f32_to_bf16(d);
      }
    }
  }
  if (dgamma) {
    for (int64_t j = 0; j < D; ++j) {
      Sum acc(mode);
      for (int64_t t = 0; t < T; ++t) {
        const float hj = bf16_to_f32(x[t * ld_x + j]) + bf16_to_f32(residual[t * ld_res + j]);
        const float gh = bf16_to_f32(g[t * ld_g + j]) * hj;
        const float term = gh * rstd[t];
        acc.add(term);
      }
      dgamma[j] = acc.value();
    }
  }
  delete[] h;
  return 0;
}

// ---- activation and weight dtypes ---------------------------------------------
// fp16 activations and bf16 / fp16 weights (RL-Kernel PR "C1: zero-centred
// RMSNorm references and CUDA kernel" checks fp16 as well as bf16; Megatron-LM
// PR "Fix the batch-invariant RMSNorm forward ...", item 1: the weight is cast
// to fp32 and only then offset by 1). Every storage type widens to fp32
// exactly; the arithmetic is that of the bf16 / fp32 functions above.

}  // extern "C"

namespace {

// IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
float f16_to_f32(uint16_t h) {
  const uint32_t sign = static_cast<uint32_t>(h & 0x8000u) << 16;
  const int e = (h >> 10) & 0x1F;
  const uint32_t frac = h & 0x3FFu;
  float mag;
  if (e == 31) {  // inf, or NaN (quieted, payload kept in the top fraction bits)
    uint32_t u = sign | 0x7F800000u | (frac << 13) | (frac ? 0x00400000u : 0u);
    float f;
    std::memcpy(&f, &u, 4);
    return f;
  }
  if (e == 0)
    mag = std::ldexp(static_cast<float>(frac), -24);          // subnormal: frac * 2^-24
  else
    mag = std::ldexp(static_cast<float>(frac | 0x400u), e - 25);  // (1024 + frac) * 2^(e-25)
  uint32_t u;
  std::memcpy(&u, &mag, 4);
  u |= sign;
  std::memcpy(&mag, &u, 4);
  return mag;
}

// Round to the nearest binary16, ties to even (the significand rounded with
// nearbyint under the default rounding mode, in exact double arithmetic);
// subnormals kept; |f| >= 65520 (halfway past the largest finite, 65504)
// becomes infinity; NaN becomes a quiet NaN of the same sign.
uint16_t f32_to_f16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  const uint16_t sign = static_cast<uint16_t>((u >> 16) & 0x8000u);
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return static_cast<uint16_t>(sign | 0x7E00u | ((a >> 13) & 0x1FFu));
  const double af = std::fabs(static_cast<double>(f));
  if (af >= 65520.0) return static_cast<uint16_t>(sign | 0x7C00u);
  if (af < std::ldexp(1.0, -14)) {  // subnormal range: m * 2^-24
    const double m = std::nearbyint(af * std::ldexp(1.0, 24));
    return static_cast<uint16_t>(sign | static_cast<uint16_t>(m));  // m = 1024 is the smallest normal
  }
  int e;
  const double fr = std::frexp(af, &e);  // af = fr * 2^e, fr in [0.5, 1)
  double sm = std::nearbyint(fr * 2048.0);  // 11-bit significand in [1024, 2048]
  if (sm == 2048.0) {
    sm = 1024.0;
    e += 1;
  }
  const int biased = e + 14;  // af = (sm / 1024) * 2^(e - 1)
  if (biased >= 31) return static_cast<uint16_t>(sign | 0x7C00u);
  return static_cast<uint16_t>(sign | (biased << 10) | (static_cast<uint32_t>(sm) - 1024u));
}

float act_to_f32(int dt, uint16_t b) { return dt == ORACLE_F16 ? f16_to_f32(b) : bf16_to_f32(b); }
uint16_t f32_to_act(int dt, float f) { return dt == ORACLE_F16 ? f32_to_f16(f) : f32_to_bf16(f); }
bool bad_act_dt(int dt) { return dt != ORACLE_BF16 && dt != ORACLE_F16; }
bool bad_weight_dt(int dt) { return dt != ORACLE_F32 && dt != ORACLE_BF16 && dt != ORACLE_F16; }

// The weight in fp32 (exact widening), then + 1.0f in fp32 when zero-centred.
float weight_eff_dt(int wdt, const void* gamma, int zc, int64_t j) {
  float w;
  if (wdt == ORACLE_F32)
    w = static_cast<const float*>(gamma)[j];
  else
    w = act_to_f32(wdt, static_cast<const uint16_t*>(gamma)[j]);
  if (zc) w = w + 1.0f;
  return w;
}

}  // namespace

extern "C" {

void oracle_f16_decode(const uint16_t* in, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f16_to_f32(in[i]);
}

void oracle_f16_encode(const float* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_f16(in[i]);
}

int oracle_rmsnorm_fwd_dt(int mode, int act_dtype, int weight_dtype, const uint16_t* x,
                          int64_t ld_x, const void* gamma, int zero_centered, float eps, int64_t T,
                          int64_t D, uint16_t* y, int64_t ld_y, float* rstd) {
  if (bad_mode(mode) || bad_act_dt(act_dtype) || bad_weight_dt(weight_dtype) || T < 0 || D <= 0 ||
      !gamma || bad_2d(x, ld_x, D) || bad_2d(y, ld_y, D))
    return -1;
  for (int64_t t = 0; t < T; ++t) {
    const uint16_t* xr = x + t * ld_x;
    Sum ss(mode);
    for (int64_t j = 0; j < D; ++j) {
      const float xf = act_to_f32(act_dtype, xr[j]);
      const float sq = xf * xf;  // exact for bf16 and fp16 inputs
      ss.add(sq);
    }
    const float mean = ss.value() / static_cast<float>(D);
    const float v = mean + eps;
    const float r = rsqrt_ref(v);
    if (rstd) rstd[t] = r;
    for (int64_t j = 0; j < D; ++j) {
      const float n = row_normed(act_to_f32(act_dtype, xr[j]), r,
                                 weight_eff_dt(weight_dtype, gamma, zero_centered, j));
      y[t * ld_y + j] = f32_to_act(act_dtype, n);
    }
  }
  return 0;
}

int oracle_rmsnorm_bwd_dx_dt(int mode, int act_dtype, int weight_dtype, const uint16_t* g,
                             int64_t ld_g, const uint16_t* x, int64_t ld_x, const float* rstd,
                             const void* gamma, int zero_centered, int64_t T, int64_t D,
                             const uint16_t* gres, int64_t ld_gres, uint16_t* dx, int64_t ld_dx) {
  if (bad_mode(mode) || bad_act_dt(act_dtype) || bad_weight_dt(weight_dtype) || T < 0 || D <= 0 ||
      !gamma || !rstd || bad_2d(g, ld_g, D) || bad_2d(x, ld_x, D) || bad_2d(dx, ld_dx, D) ||
      (gres && ld_gres < D))
    return -1;
  for (int64_t t = 0; t < T; ++t) {
    const uint16_t* gr = g + t * ld_g;
    const uint16_t* xr = x + t * ld_x;
    const float r = rstd[t];
    Sum s(mode);
    for (int64_t i = 0; i < D; ++i) {
      const float gw = act_to_f32(act_dtype, gr[i]) *
                       weight_eff_dt(weight_dtype, gamma, zero_centered, i);
      const float term = gw * act_to_f32(act_dtype, xr[i]);
      s.add(term);
    }
    const float r2 = r * r;
    const float r3 = r2 * r;
    const float r3s = r3 * s.value();
    const float c = r3s / static_cast<float>(D);
    for (int64_t k = 0; k < D; ++k) {
      const float w = weight_eff_dt(weight_dtype, gamma, zero_centered, k);
      const float gw = act_to_f32(act_dtype, gr[k]) * w;
      const float t1 = gw * r;
      const float t2 = act_to_f32(act_dtype, xr[k]) * c;
      float d = t1 - t2;
      if (gres) d = d + act_to_f32(act_dtype, gres[t * ld_gres + k]);
      dx[t * ld_dx + k] = f32_to_act(act_dtype, d);
    }
  }
  return 0;
}

int oracle_rmsnorm_dgamma_dt(int mode, int act_dtype, const uint16_t* g, int64_t ld_g,
                             const uint16_t* x, int64_t ld_x, const float* rstd, int64_t T,
                             int64_t ncols, float* dgamma) {
  if (bad_mode(mode) || bad_act_dt(act_dtype) || T < 0 || ncols <= 0 || !dgamma ||
      bad_2d(g, ld_g, ncols) || bad_2d(x, ld_x, ncols) || (T > 0 && !rstd))
    return -1;
  for (int64_t j = 0; j < ncols; ++j) {
    Sum acc(mode);
    for (int64_t t = 0; t < T; ++t) {
      const float gx = act_to_f32(act_dtype, g[t * ld_g + j]) * act_to_f32(act_dtype, x[t * ld_x + j]);
      const float term = gx * rstd[t];
      acc.add(term);
    }
    dgamma[j] = acc.value();
  }
  return 0;
}

// ---- gated norm and fused add-norm in other storage types ----------------------
// The same definitions as oracle_rmsnorm_gated_* and oracle_rmsnorm_add_*
// above, with activations (x, z, g, residual, gradients, outputs) stored as
// bf16 or fp16 and weights as fp32, bf16 or fp16. Every storage type widens to
// fp32 exactly; the gated cast convention rounds to the activations' type
// ("cast to the input dtype", RL-Kernel PR "C1: zero-centred RMSNorm
// references and CUDA kernel", gated-norm conventions).

static float round_act(int dt, float v) { return act_to_f32(dt, f32_to_act(dt, v)); }

// rstd of a row of stored activations: squares of the widened values (exact
// for bf16 and fp16) summed in the mode's order.
static float row_rstd_dt(int mode, int dt, const uint16_t* xr, int64_t D, float eps) {
  Sum ss(mode);
  for (int64_t j = 0; j < D; ++j) {
    const float xf = act_to_f32(dt, xr[j]);
    const float sq = xf * xf;
    ss.add(sq);
  }
  const float mean = ss.value() / static_cast<float>(D);
  const float v = mean + eps;
  return rsqrt_ref(v);
}

int oracle_rmsnorm_gated_fwd_dt(int mode, int act_dtype, int weight_dtype, int activation,
                                int convention, const uint16_t* x, int64_t ld_x,
                                const uint16_t* z, int64_t ld_z, const void* gamma,
                                int zero_centered, float eps, int64_t T, int64_t D, uint16_t* out,
                                int64_t ld_out, float* rstd) {
  if (bad_mode(mode) || bad_act_dt(act_dtype) || bad_weight_dt(weight_dtype) ||
      bad_act(activation) || (convention != ORACLE_GATED_FP32 && convention != ORACLE_GATED_CAST) ||
      T < 0 || D <= 0 || !gamma || bad_2d(x, ld_x, D) || bad_2d(z, ld_z, D) ||
      bad_2d(out, ld_out, D))
    return -1;
  for (int64_t t = 0; t < T; ++t) {
    const uint16_t* xr = x + t * ld_x;
    const float r = row_rstd_dt(mode, act_dtype, xr, D, eps);
    if (rstd) rstd[t] = r;
    for (int64_t j = 0; j < D; ++j) {
      const float w = weight_eff_dt(weight_dtype, gamma, zero_centered, j);
      const float a = static_cast<float>(gate_d(activation, act_to_f32(act_dtype, z[t * ld_z + j])));
      float n = act_to_f32(act_dtype, xr[j]) * r;
      if (convention == ORACLE_GATED_CAST) n = round_act(act_dtype, n);
      float nw = n * w;
      if (convention == ORACLE_GATED_CAST) nw = round_act(act_dtype, nw);
      const float o = nw * a;
      out[t * ld_out + j] = f32_to_act(act_dtype, o);
    }
  }
  return 0;
}

int oracle_rmsnorm_gated_bwd_dt(int mode, int act_dtype, int weight_dtype, int activation,
                                const uint16_t* g, int64_t ld_g, const uint16_t* x, int64_t ld_x,
                                const uint16_t* z, int64_t ld_z, const float* rstd,
                                const void* gamma, int zero_centered, int64_t T, int64_t D,
                                uint16_t* dx, int64_t ld_dx, uint16_t* dz, int64_t ld_dz) {
  if (bad_mode(mode) || bad_act_dt(act_dtype) || bad_weight_dt(weight_dtype) ||
      bad_act(activation) || T < 0 || D <= 0 || !gamma || !rstd || bad_2d(g, ld_g, D) ||
      bad_2d(x, ld_x, D) || bad_2d(z, ld_z, D) || (!dx && !dz) || (dx && ld_dx < D) ||
      (dz && ld_dz < D))
    return -1;
  for (int64_t t = 0; t < T; ++t) {
    const uint16_t* gr = g + t * ld_g;
    const uint16_t* xr = x + t * ld_x;
    const uint16_t* zr = z + t * ld_z;
    const float r = rstd[t];
    Sum s(mode);
    for (int64_t i = 0; i < D; ++i) {
      const float a = static_cast<float>(gate_d(activation, act_to_f32(act_dtype, zr[i])));
      const float gn = act_to_f32(act_dtype, gr[i]) * a;
      const float gw = gn * weight_eff_dt(weight_dtype, gamma, zero_centered, i);
      const float term = gw * act_to_f32(act_dtype, xr[i]);
      s.add(term);
    }
    const float r2 = r * r;
    const float r3 = r2 * r;
    const float r3s = r3 * s.value();
    const float c = r3s / static_cast<float>(D);
    for (int64_t k = 0; k < D; ++k) {
      const float w = weight_eff_dt(weight_dtype, gamma, zero_centered, k);
      const float xf = act_to_f32(act_dtype, xr[k]);
      const float gf = act_to_f32(act_dtype, gr[k]);
      const double zd = act_to_f32(act_dtype, zr[k]);
      const float a = static_cast<float>(gate_d(activation, zd));
      const float da = static_cast<float>(gate_grad_d(activation, zd));
      if (dz) {
        const float n = xf * r;
        const float nw = n * w;
        const float gnw = gf * nw;
        dz[t * ld_dz + k] = f32_to_act(act_dtype, gnw * da);
      }
      if (dx) {
        const float gn = gf * a;
        const float gw = gn * w;
        const float t1 = gw * r;
        const float t2 = xf * c;
        dx[t * ld_dx + k] = f32_to_act(act_dtype, t1 - t2);
      }
    }
  }
  return 0;
}

int oracle_rmsnorm_gated_dgamma_dt(int mode, int act_dtype, int activation, const uint16_t* g,
                                   int64_t ld_g, const uint16_t* x, int64_t ld_x,
                                   const uint16_t* z, int64_t ld_z, const float* rstd, int64_t T,
                                   int64_t ncols, float* dgamma) {
  if (bad_mode(mode) || bad_act_dt(act_dtype) || bad_act(activation) || T < 0 || ncols <= 0 ||
      !dgamma || bad_2d(g, ld_g, ncols) || bad_2d(x, ld_x, ncols) || bad_2d(z, ld_z, ncols) ||
      (T > 0 && !rstd))
    return -1;
  for (int64_t j = 0; j < ncols; ++j) {
    Sum acc(mode);
    for (int64_t t = 0; t < T; ++t) {
      const float a =
          static_cast<float>(gate_d(activation, act_to_f32(act_dtype, z[t * ld_z + j])));
      const float gn = act_to_f32(act_dtype, g[t * ld_g + j]) * a;
      const float gx = gn * act_to_f32(act_dtype, x[t * ld_x + j]);
      const float term = gx * rstd[t];
      acc.add(term);
    }
    dgamma[j] = acc.value();
  }
  return 0;
}

int oracle_rmsnorm_add_fwd_dt(int mode, int act_dtype, int weight_dtype, const uint16_t* x,
                              int64_t ld_x, const uint16_t* residual, int64_t ld_res,
                              const void* gamma, int zero_centered, float eps, int64_t T, int64_t D,
                              uint16_t* y, int64_t ld_y, uint16_t* residual_out, int64_t ld_rout,
                              float* rstd) {
  if (bad_mode(mode) || bad_act_dt(act_dtype) || bad_weight_dt(weight_dtype) || T < 0 || D <= 0 ||
      !gamma || bad_2d(x, ld_x, D) || bad_2d(residual, ld_res, D) || bad_2d(y, ld_y, D) ||
      bad_2d(residual_out, ld_rout, D))
    return -1;
  float* h = new float[static_cast<size_t>(D)];
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t j = 0; j < D; ++j)
      h[j] = act_to_f32(act_dtype, x[t * ld_x + j]) + act_to_f32(act_dtype, residual[t * ld_res + j]);
    Sum ss(mode);
    for (int64_t j = 0; j < D; ++j) {
      const float sq = h[j] * h[j];
      ss.add(sq);
    }
    const float mean = ss.value() / static_cast<float>(D);
    const float r = rsqrt_ref(mean + eps);
    if (rstd) rstd[t] = r;
    for (int64_t j = 0; j < D; ++j) {
      const float n = row_normed(h[j], r, weight_eff_dt(weight_dtype, gamma, zero_centered, j));
      y[t * ld_y + j] = f32_to_act(act_dtype, n);
      residual_out[t * ld_rout + j] = f32_to_act(act_dtype, h[j]);
    }
  }
  delete[] h;
  return 0;
}

int oracle_rmsnorm_add_bwd_dt(int mode, int act_dtype, int weight_dtype, const uint16_t* g,
                              int64_t ld_g, const uint16_t* x, int64_t ld_x,
                              const uint16_t* residual, int64_t ld_res, const float* rstd,
                              const void* gamma, int zero_centered, int64_t T, int64_t D,
                              const uint16_t* g_rout, int64_t ld_gro, uint16_t* dh, int64_t ld_dh,
                              float* dgamma) {
  if (bad_mode(mode) || bad_act_dt(act_dtype) || bad_weight_dt(weight_dtype) || T < 0 || D <= 0 ||
      !gamma || (T > 0 && !rstd) || bad_2d(g, ld_g, D) || bad_2d(x, ld_x, D) ||
      bad_2d(residual, ld_res, D) || (!dh && !dgamma) || (dh && ld_dh < D) ||
      (g_rout && ld_gro < D))
    return -1;
  auto h_of = [&](int64_t t, int64_t j) {
    return act_to_f32(act_dtype, x[t * ld_x + j]) + act_to_f32(act_dtype, residual[t * ld_res + j]);
  };
  if (dh) {
    for (int64_t t = 0; t < T; ++t) {
      const uint16_t* gr = g + t * ld_g;
      const float r = rstd[t];
      Sum s(mode);
      for (int64_t i = 0; i < D; ++i) {
        const float gw = act_to_f32(act_dtype, gr[i]) *
                         weight_eff_dt(weight_dtype, gamma, zero_centered, i);
        const float term = gw * h_of(t, i);
        s.add(term);
      }
      const float r2 = r * r;
      const float r3 = r2 * r;
      const float r3s = r3 * s.value();
      const float c = r3s / static_cast<float>(D);
      for (int64_t k = 0; k < D; ++k) {
        const float gw = act_to_f32(act_dtype, gr[k]) *
                         weight_eff_dt(weight_dtype, gamma, zero_centered, k);
        const float t1 = gw * r;
        const float t2 = h_of(t, k) * c;
        float d = t1 - t2;
        if (g_rout) d = d + act_to_f32(act_dtype, g_rout[t * ld_gro + k]);
        dh[t * ld_dh + k] = f32_to_act(act_dtype, d);
      }
    }
  }
  if (dgamma) {
    for (int64_t j = 0; j < D; ++j) {
      Sum acc(mode);
      for (int64_t t = 0; t < T; ++t) {
        const float gh = act_to_f32(act_dtype, g[t * ld_g + j]) * h_of(t, j);
        const float term = gh * rstd[t];
        acc.add(term);
      }
      dgamma[j] = acc.value();
    }
  }
  return 0;
}

// ---- batch-invariant GEMM ----------------------------------------------------
// TransformerEngine issue "Expose Batch Invariant Kernels", point 3: BF16,
// Y = X @ W.T over contiguous 2-D operands. The plain definition: each
// output is the dot product of a row of X and a row of W; here it is summed
// in double in ascending k (the products of bf16 values are exact in double),
// rounded to fp32 and then to bf16.

int oracle_gemm_xwt(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw, int64_t M,
                    int64_t N, int64_t K, uint16_t* Y, int64_t ldy, double* Y_exact) {
  if (M < 0 || N < 0 || K < 0 || !X || !W || !Y || ldx < K || ldw < K || ldy < N) return -1;
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t j = 0; j < N; ++j) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k)
        acc += static_cast<double>(bf16_to_f32(X[i * ldx + k])) *
               static_cast<double>(bf16_to_f32(W[j * ldw + k]));
      if (Y_exact) Y_exact[i * N + j] = acc;
      Y[i * ldy + j] = f32_to_bf16(static_cast<float>(acc));
    }
  }
  return 0;
}

// ---- exact double forms ----------------------------------------------------

static double weight_eff_d(const double* gamma, int zc, int64_t j) {
  return zc ? gamma[j] + 1.0 : gamma[j];
}

static double row_rstd_d(const double* xr, int64_t D, double eps) {
  double ss = 0.0;
  for (int64_t j = 0; j < D; ++j) ss += xr[j] * xr[j];
  return 1.0 / std::sqrt(ss / static_cast<double>(D) + eps);
}

int oracle_rmsnorm_fwd_f64(const double* x, const double* gamma, int zero_centered,
                           double eps, int64_t T, int64_t D, double* y, double* rstd) {
  if (!x || !gamma || !y || T < 0 || D <= 0) return -1;
  const int zc_fwd = (g_mutation == 1) ? 0 : zero_centered;
  for (int64_t t = 0; t < T; ++t) {
    const double r = row_rstd_d(x + t * D, D, eps);
    if (rstd) rstd[t] = r;
    for (int64_t j = 0; j < D; ++j)
      y[t * D + j] = x[t * D + j] * r * weight_eff_d(gamma, zc_fwd, j);
  }
  return 0;
}

int oracle_rmsnorm_gated_fwd_f64(const double* x, const double* z, const double* gamma,
                                 int zero_centered, double eps, int64_t T, int64_t D,
                                 double* out) {
  if (!x || !z || !gamma || !out || T < 0 || D <= 0) return -1;
  const int zc_fwd = (g_mutation == 1) ? 0 : zero_centered;
  for (int64_t t = 0; t < T; ++t) {
    const double r = row_rstd_d(x + t * D, D, eps);
    for (int64_t j = 0; j < D; ++j)
      out[t * D + j] =
          x[t * D + j] * r * weight_eff_d(gamma, zc_fwd, j) * silu_d(z[t * D + j]);
  }
  return 0;
}

int oracle_rmsnorm_gated_fwd_ex_f64(int activation, const double* x, const double* z,
                                    const double* gamma, int zero_centered, double eps, int64_t T,
                                    int64_t D, double* out) {
  if (bad_act(activation) || !x || !z || !gamma || !out || T < 0 || D <= 0) return -1;
  const int zc_fwd = (g_mutation == 1) ? 0 : zero_centered;
  for (int64_t t = 0; t < T; ++t) {
    const double r = row_rstd_d(x + t * D, D, eps);
    for (int64_t j = 0; j < D; ++j)
      out[t * D + j] =
          x[t * D + j] * r * weight_eff_d(gamma, zc_fwd, j) * gate_d(activation, z[t * D + j]);
  }
  return 0;
}

// L = sum g * out with out = (x r w) a(z): dz = g x r w a'(z); the norm sees
// the upstream gradient gn = g a(z), and dx, dgamma follow from the plain
// backward with gn in place of g.
int oracle_rmsnorm_gated_bwd_f64(int activation, const double* g, const double* x, const double* z,
                                 const double* gamma, int zero_centered, double eps, int64_t T,
                                 int64_t D, double* dx, double* dz, double* dgamma) {
  if (bad_act(activation) || !g || !x || !z || !gamma || T < 0 || D <= 0) return -1;
  double* gn = new double[static_cast<size_t>(T * D)];
  for (int64_t i = 0; i < T * D; ++i) gn[i] = g[i] * gate_d(activation, z[i]);
  if (dz) {
    for (int64_t t = 0; t < T; ++t) {
      const double r = row_rstd_d(x + t * D, D, eps);
      for (int64_t k = 0; k < D; ++k)
        dz[t * D + k] = g[t * D + k] * x[t * D + k] * r * weight_eff_d(gamma, zero_centered, k) *
                        gate_grad_d(activation, z[t * D + k]);
    }
  }
  int rc = 0;
  if (dx || dgamma)
    rc = oracle_rmsnorm_bwd_f64(gn, x, gamma, zero_centered, eps, T, D, nullptr, dx, dgamma);
  delete[] gn;
  return rc;
}

int oracle_rmsnorm_bwd_f64(const double* g, const double* x, const double* gamma,
                           int zero_centered, double eps, int64_t T, int64_t D,
                           const double* gres, double* dx, double* dgamma) {
  if (!g || !x || !gamma || T < 0 || D <= 0 || (!dx && !dgamma)) return -1;
  if (dgamma)
    for (int64_t j = 0; j < D; ++j) dgamma[j] = 0.0;
  for (int64_t t = 0; t < T; ++t) {
    const double* gr = g + t * D;
    const double* xr = x + t * D;
    const double r = row_rstd_d(xr, D, eps);
    // s = sum_i g_i x_i w_i; dr/dx_k = -r^3 x_k / D.
    double s = 0.0;
    for (int64_t i = 0; i < D; ++i) s += gr[i] * xr[i] * weight_eff_d(gamma, zero_centered, i);
    for (int64_t k = 0; k < D; ++k) {
      const double w = weight_eff_d(gamma, zero_centered, k);
      double second = r * r * r * xr[k] / static_cast<double>(D) * s;
      if (g_mutation == 2) second *= w;
      if (dx) dx[t * D + k] = gr[k] * w * r - second + (gres ? gres[t * D + k] : 0.0);
      if (dgamma) dgamma[k] += gr[k] * xr[k] * r;
    }
  }
  return 0;
}

// Fused add-RMSNorm in double: h = x + residual exactly, y = h r w; the
// residual output is h. For L = sum g * y + sum g_rout * h, the gradient
// with respect to h (and so to x and to residual alike) is the plain
// backward at h plus g_rout.
int oracle_rmsnorm_add_fwd_f64(const double* x, const double* residual, const double* gamma,
                               int zero_centered, double eps, int64_t T, int64_t D, double* y,
                               double* h_out, double* rstd) {
  if (!x || !residual || !gamma || !y || T < 0 || D <= 0) return -1;
  double* h = new double[static_cast<size_t>(T * D)];
  for (int64_t i = 0; i < T * D; ++i) h[i] = x[i] + residual[i];
  const int rc = oracle_rmsnorm_fwd_f64(h, gamma, zero_centered, eps, T, D, y, rstd);
  if (h_out)
    for (int64_t i = 0; i < T * D; ++i) h_out[i] = h[i];
  delete[] h;
  return rc;
}

int oracle_rmsnorm_add_bwd_f64(const double* g, const double* x, const double* residual,
                               const double* gamma, int zero_centered, double eps, int64_t T,
                               int64_t D, const double* g_rout, double* dh, double* dgamma) {
  if (!g || !x || !residual || !gamma || T < 0 || D <= 0 || (!dh && !dgamma)) return -1;
  double* h = new double[static_cast<size_t>(T * D)];
  for (int64_t i = 0; i < T * D; ++i) h[i] = x[i] + residual[i];
  const int rc = oracle_rmsnorm_bwd_f64(g, h, gamma, zero_centered, eps, T, D, g_rout, dh, dgamma);
  delete[] h;
  return rc;
}

}  // extern "C"
