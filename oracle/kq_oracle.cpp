// kq_oracle.cpp — fp64 CPU oracle of the KroQuant online activation quantizer.
// TEST INFRASTRUCTURE ONLY: see kq_oracle.h for the sources and the conventions.
// Built with -O2 -ffp-contract=off so that every product and sum is rounded
// separately, exactly as written.
#include "kq_oracle.h"

#include <cmath>
#include <cstring>
#include <thread>
#include <vector>
#include <algorithm>

namespace {

constexpr int kBlk = 32;       // channels per block and per MX block [ABS], [MX]
constexpr int kFactors = 5;    // 2^5 = 32 [POD]

// E2M1 magnitudes, indexed by the 3-bit magnitude code. [MX]
constexpr double kGrid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

int threads_for(int nthreads, int64_t rows) {
  int n = nthreads > 0 ? nthreads : (int)std::thread::hardware_concurrency();
  if (n < 1) n = 1;
  if ((int64_t)n > rows) n = (int)std::max<int64_t>(rows, 1);
  return n;
}

// Run body(r0, r1) over [0, rows) split into contiguous row ranges.
template <class F>
void parallel_rows(int64_t rows, int nthreads, F body) {
  int n = threads_for(nthreads, rows);
  if (n <= 1) { body(0, rows); return; }
  std::vector<std::thread> pool;
  int64_t per = (rows + n - 1) / n;
  for (int i = 0; i < n; ++i) {
    int64_t r0 = i * per, r1 = std::min(rows, r0 + per);
    if (r0 >= r1) break;
    pool.emplace_back([=] { body(r0, r1); });
  }
  for (auto& t : pool) t.join();
}

bool bad_shape(int64_t rows, int64_t d, int64_t ldx) {
  return rows < 0 || d <= 0 || d % kBlk != 0 || ldx < d;
}

}  // namespace

extern "C" {

void oq_factor(double l, double u, double v, double F[4]) {
  // L = [[1,0],[l,1]], U = [[u,v],[0,1/u]]; F = L*U written out as a 2x2 product.
  const double L[4] = {1.0, 0.0, l, 1.0};
  const double U[4] = {u, v, 0.0, 1.0 / u};
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j)
      F[2 * i + j] = L[2 * i + 0] * U[0 * 2 + j] + L[2 * i + 1] * U[1 * 2 + j];
}

void oq_factor_inverse(double l, double u, double v, double Finv[4]) {
  // (L*U)^-1 = U^-1 * L^-1 with U^-1 = [[1/u, -v],[0, u]] and L^-1 = [[1,0],[-l,1]].
  const double Ui[4] = {1.0 / u, -v, 0.0, u};
  const double Li[4] = {1.0, 0.0, -l, 1.0};
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j)
      Finv[2 * i + j] = Ui[2 * i + 0] * Li[0 * 2 + j] + Ui[2 * i + 1] * Li[1 * 2 + j];
}

void oq_kron(const double* A, int ar, int ac, const double* B, int br, int bc, double* C) {
  // (A (x) B)[i*br + r][j*bc + s] = A[i][j] * B[r][s]
  const int cc = ac * bc;
  for (int i = 0; i < ar; ++i)
    for (int j = 0; j < ac; ++j)
      for (int r = 0; r < br; ++r)
        for (int s = 0; s < bc; ++s)
          C[(int64_t)(i * br + r) * cc + (j * bc + s)] = A[i * ac + j] * B[r * bc + s];
}

int oq_expand(const float* params, int64_t nb, int inverse, double* T) {
  if (!params || !T || nb < 0) return -1;
  for (int64_t b = 0; b < nb; ++b) {
    double F[kFactors][4];
    for (int k = 0; k < kFactors; ++k) {
      const float* p = params + (b * kFactors + k) * 3;
      if (inverse) oq_factor_inverse(p[0], p[1], p[2], F[k]);
      else         oq_factor(p[0], p[1], p[2], F[k]);
    }
    // T_b = F1 (x) (F2 (x) (F3 (x) (F4 (x) F5))), built from the right.
    std::vector<double> acc(F[kFactors - 1], F[kFactors - 1] + 4), next;
    int n = 2;
    for (int k = kFactors - 2; k >= 0; --k) {
      next.assign((size_t)(2 * n) * (2 * n), 0.0);
      oq_kron(F[k], 2, 2, acc.data(), n, n, next.data());
      acc.swap(next);
      n *= 2;
    }
    std::memcpy(T + b * kBlk * kBlk, acc.data(), sizeof(double) * kBlk * kBlk);
  }
  return 0;
}

double oq_det(const double* A, int n) {
  std::vector<double> M(A, A + (size_t)n * n);
  double det = 1.0;
  for (int c = 0; c < n; ++c) {
    int p = c;
    for (int r = c + 1; r < n; ++r)
      if (std::fabs(M[(size_t)r * n + c]) > std::fabs(M[(size_t)p * n + c])) p = r;
    if (M[(size_t)p * n + c] == 0.0) return 0.0;
    if (p != c) {
      for (int j = 0; j < n; ++j) std::swap(M[(size_t)p * n + j], M[(size_t)c * n + j]);
      det = -det;
    }
    const double piv = M[(size_t)c * n + c];
    det *= piv;
    for (int r = c + 1; r < n; ++r) {
      const double f = M[(size_t)r * n + c] / piv;
      for (int j = c; j < n; ++j) M[(size_t)r * n + j] -= f * M[(size_t)c * n + j];
    }
  }
  return det;
}

double oq_load(const void* x, int dtype, int64_t idx) {
  if (dtype == OQ_BF16) {
    // bf16 is the top half of an fp32: widening is exact.
    uint32_t bits = (uint32_t)((const uint16_t*)x)[idx] << 16;
    float f;
    std::memcpy(&f, &bits, 4);
    return (double)f;
  }
  return (double)((const float*)x)[idx];
}

int oq_transform_dense(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                       const double* T, double* y) {
  if (rows == 0 && !bad_shape(rows, d, ldx)) return 0;
  if (!x || !T || !y || bad_shape(rows, d, ldx) || (dtype != OQ_BF16 && dtype != OQ_FP32))
    return -1;
  const int64_t nb = d / kBlk;
  for (int64_t t = 0; t < rows; ++t)
    for (int64_t b = 0; b < nb; ++b) {
      double xb[kBlk];
      for (int j = 0; j < kBlk; ++j) xb[j] = oq_load(x, dtype, t * ldx + b * kBlk + j);
      const double* Tb = T + b * kBlk * kBlk;
      for (int i = 0; i < kBlk; ++i) {
        double acc = 0.0;
        for (int j = 0; j < kBlk; ++j) acc += Tb[i * kBlk + j] * xb[j];
        y[t * d + b * kBlk + i] = acc;
      }
    }
  return 0;
}

int oq_transform_factored(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                          const float* params, double* y) {
  if (!x || !params || !y || bad_shape(rows, d, ldx) || (dtype != OQ_BF16 && dtype != OQ_FP32))
    return -1;
  const int64_t nb = d / kBlk;
  for (int64_t t = 0; t < rows; ++t)
    for (int64_t b = 0; b < nb; ++b) {
      double v[kBlk];
      for (int j = 0; j < kBlk; ++j) v[j] = oq_load(x, dtype, t * ldx + b * kBlk + j);
      for (int k = 0; k < kFactors; ++k) {
        const float* p = params + (b * kFactors + k) * 3;
        double F[4];
        oq_factor(p[0], p[1], p[2], F);
        const int stride = 1 << (kFactors - 1 - k);  // F1 on bit 4 ... F5 on bit 0
        for (int i = 0; i < kBlk; ++i) {
          if (i & stride) continue;
          const double a = v[i], c = v[i + stride];
          v[i] = F[0] * a + F[1] * c;
          v[i + stride] = F[2] * a + F[3] * c;
        }
      }
      for (int i = 0; i < kBlk; ++i) y[t * d + b * kBlk + i] = v[i];
    }
  return 0;
}

int oq_scale_exp(double amax) {
  if (!std::isfinite(amax)) return 128;
  if (amax == 0.0) return -127;
  int E;
  (void)std::frexp(std::fabs(amax), &E);  // amax = f * 2^E, f in [0.5, 1)
  int e = (E - 1) - 2;                     // floor(log2 amax) - emax(E2M1)
  return std::min(127, std::max(-127, e));
}

int oq_e2m1_code(double y, int e) {
  if (std::isnan(y)) return 0;
  const int sign = std::signbit(y) ? 8 : 0;
  const double r = std::ldexp(std::fabs(y), -e);  // |y| / 2^e, exact
  // Nearest grid value; a midpoint goes to the even code; beyond 6 saturates to 6.
  int m;
  if (r <= 0.25) m = 0;
  else if (r < 0.75) m = 1;
  else if (r <= 1.25) m = 2;
  else if (r < 1.75) m = 3;
  else if (r <= 2.5) m = 4;
  else if (r < 3.5) m = 5;
  else if (r <= 5.0) m = 6;
  else m = 7;
  return sign | m;
}

double oq_e2m1_value(int code, int e) {
  const double mag = std::ldexp(kGrid[code & 7], e);
  return (code & 8) ? -mag : mag;
}

int oq_dequantize(const uint8_t* q, int64_t ldq, const uint8_t* s, int64_t lds, int64_t rows,
                  int64_t d, double* out) {
  if (rows == 0 && d > 0 && d % kBlk == 0) return 0;
  if (!q || !s || !out || rows < 0 || d <= 0 || d % kBlk != 0 || ldq < d / 2 || lds < d / kBlk)
    return -1;
  for (int64_t t = 0; t < rows; ++t)
    for (int64_t c = 0; c < d; ++c) {
      const int S = s[t * lds + c / kBlk];
      const uint8_t byte = q[t * ldq + c / 2];
      const int code = (c % 2 == 0) ? (byte & 0xF) : (byte >> 4);
      out[t * d + c] = S == 0xFF ? std::nan("") : oq_e2m1_value(code, S - 127);
    }
  return 0;
}

int oq_encode(const double* y, int64_t rows, int64_t d, uint8_t* q, int64_t ldq,
              uint8_t* s, int64_t lds) {
  if (rows == 0 && d > 0 && d % kBlk == 0) return 0;
  if (!y || !q || !s || rows < 0 || d <= 0 || d % kBlk != 0 || ldq < d / 2 || lds < d / kBlk)
    return -1;
  const int64_t nb = d / kBlk;
  for (int64_t t = 0; t < rows; ++t)
    for (int64_t b = 0; b < nb; ++b) {
      const double* yb = y + t * d + b * kBlk;
      double amax = 0.0;
      bool finite = true;
      for (int i = 0; i < kBlk; ++i) {
        if (!std::isfinite(yb[i])) finite = false;
        amax = std::max(amax, std::fabs(yb[i]));
      }
      uint8_t* qb = q + t * ldq + b * (kBlk / 2);
      if (!finite) {
        s[t * lds + b] = 0xFF;
        std::memset(qb, 0, kBlk / 2);
        continue;
      }
      const int e = oq_scale_exp(amax);
      s[t * lds + b] = (uint8_t)(e + 127);
      for (int i = 0; i < kBlk; i += 2)
        qb[i / 2] = (uint8_t)(oq_e2m1_code(yb[i], e) | (oq_e2m1_code(yb[i + 1], e) << 4));
    }
  return 0;
}

int oq_quantize(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                const float* params, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds,
                double* y_out, int nthreads) {
  if (!x || !params || !q || !s || bad_shape(rows, d, ldx) ||
      (dtype != OQ_BF16 && dtype != OQ_FP32) || ldq < d / 2 || lds < d / kBlk)
    return -1;
  const int64_t nb = d / kBlk;
  std::vector<double> T((size_t)nb * kBlk * kBlk);
  oq_expand(params, nb, 0, T.data());
  int rc = 0;
  parallel_rows(rows, nthreads, [&](int64_t r0, int64_t r1) {
    const int64_t n = r1 - r0;
    std::vector<double> ybuf;
    double* y = y_out ? y_out + r0 * d : (ybuf.resize((size_t)n * d), ybuf.data());
    const uint8_t* base = (const uint8_t*)x + r0 * ldx * (dtype == OQ_BF16 ? 2 : 4);
    if (oq_transform_dense(base, dtype, n, d, ldx, T.data(), y) != 0 ||
        oq_encode(y, n, d, q + r0 * ldq, ldq, s + r0 * lds, lds) != 0)
      rc = -1;
  });
  return rc;
}

int oq_sq_quantize(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                   const float* mult, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds,
                   double* y_out, int nthreads) {
  if (!x || !mult || !q || !s || bad_shape(rows, d, ldx) ||
      (dtype != OQ_BF16 && dtype != OQ_FP32) || ldq < d / 2 || lds < d / kBlk)
    return -1;
  int rc = 0;
  parallel_rows(rows, nthreads, [&](int64_t r0, int64_t r1) {
    const int64_t n = r1 - r0;
    std::vector<double> ybuf;
    double* y = y_out ? y_out + r0 * d : (ybuf.resize((size_t)n * d), ybuf.data());
    for (int64_t t = 0; t < n; ++t)
      for (int64_t c = 0; c < d; ++c)
        y[t * d + c] = oq_load(x, dtype, (r0 + t) * ldx + c) * (double)mult[c];
    if (oq_encode(y, n, d, q + r0 * ldq, ldq, s + r0 * lds, lds) != 0) rc = -1;
  });
  return rc;
}

int oq_hadamard_quantize(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                         uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds, double* y_out,
                         int nthreads) {
  if (!x || !q || !s || bad_shape(rows, d, ldx) || (dtype != OQ_BF16 && dtype != OQ_FP32) ||
      ldq < d / 2 || lds < d / kBlk)
    return -1;
  // the Sylvester matrix by its closed form (entries +-1); the 1/sqrt(32) scale is
  // applied to the finished sum, so an exact cancellation stays +0 as in exact
  // arithmetic (the sign of zero decides a code bit)
  double H[kBlk][kBlk];
  const double norm = 1.0 / std::sqrt((double)kBlk);
  for (int i = 0; i < kBlk; ++i)
    for (int j = 0; j < kBlk; ++j) H[i][j] = (__builtin_popcount(i & j) & 1) ? -1.0 : 1.0;
  int rc = 0;
  parallel_rows(rows, nthreads, [&](int64_t r0, int64_t r1) {
    const int64_t n = r1 - r0;
    std::vector<double> ybuf;
    double* y = y_out ? y_out + r0 * d : (ybuf.resize((size_t)n * d), ybuf.data());
    for (int64_t t = 0; t < n; ++t)
      for (int64_t b = 0; b < d / kBlk; ++b) {
        double xb[kBlk];
        for (int j = 0; j < kBlk; ++j) xb[j] = oq_load(x, dtype, (r0 + t) * ldx + b * kBlk + j);
        for (int i = 0; i < kBlk; ++i) {
          double acc = 0.0;
          for (int j = 0; j < kBlk; ++j) acc += H[i][j] * xb[j];
          y[t * d + b * kBlk + i] = acc * norm;
        }
      }
    if (oq_encode(y, n, d, q + r0 * ldq, ldq, s + r0 * lds, lds) != 0) rc = -1;
  });
  return rc;
}

int oq_norm_quantize(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                     const float* shift, const float* scale, int64_t rows_per_sample, double eps,
                     const float* params, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds,
                     double* h_out, double* y_out, int nthreads) {
  if (!x || !params || !q || !s || bad_shape(rows, d, ldx) ||
      (dtype != OQ_BF16 && dtype != OQ_FP32) || ldq < d / 2 || lds < d / kBlk ||
      rows_per_sample < 1 || !(eps >= 0.0))
    return -1;
  const int64_t nb = d / kBlk;
  std::vector<double> T((size_t)nb * kBlk * kBlk);
  oq_expand(params, nb, 0, T.data());
  int rc = 0;
  parallel_rows(rows, nthreads, [&](int64_t r0, int64_t r1) {
    const int64_t n = r1 - r0;
    std::vector<double> hbuf, ybuf;
    double* h = h_out ? h_out + r0 * d : (hbuf.resize((size_t)n * d), hbuf.data());
    double* y = y_out ? y_out + r0 * d : (ybuf.resize((size_t)n * d), ybuf.data());
    for (int64_t t = 0; t < n; ++t) {
      const int64_t row = r0 + t;
      double* hr = h + t * d;
      for (int64_t c = 0; c < d; ++c) hr[c] = oq_load(x, dtype, row * ldx + c);
      // two-pass mean and (biased) variance
      double mu = 0.0;
      for (int64_t c = 0; c < d; ++c) mu += hr[c];
      mu /= (double)d;
      double var = 0.0;
      for (int64_t c = 0; c < d; ++c) var += (hr[c] - mu) * (hr[c] - mu);
      var /= (double)d;
      const double rstd = 1.0 / std::sqrt(var + eps);
      const int64_t g = row / rows_per_sample;
      for (int64_t c = 0; c < d; ++c) {
        const double sc = scale ? (double)scale[g * d + c] : 0.0;
        const double sh = shift ? (double)shift[g * d + c] : 0.0;
        hr[c] = (hr[c] - mu) * rstd * (1.0 + sc) + sh;
      }
      // y_b = T_b h_b
      for (int64_t b = 0; b < nb; ++b) {
        const double* Tb = T.data() + b * kBlk * kBlk;
        for (int i = 0; i < kBlk; ++i) {
          double acc = 0.0;
          for (int j = 0; j < kBlk; ++j) acc += Tb[i * kBlk + j] * hr[b * kBlk + j];
          y[t * d + b * kBlk + i] = acc;
        }
      }
    }
    if (oq_encode(y, n, d, q + r0 * ldq, ldq, s + r0 * lds, lds) != 0) rc = -1;
  });
  return rc;
}

int oq_weight_transform(const void* w, int dtype, int64_t rows, int64_t d, int64_t ldw,
                        const float* params, double* w_out) {
  if (rows == 0 && !bad_shape(rows, d, ldw)) return 0;
  if (!w || !params || !w_out || bad_shape(rows, d, ldw) || (dtype != OQ_BF16 && dtype != OQ_FP32))
    return -1;
  const int64_t nb = d / kBlk;
  std::vector<double> Ti((size_t)nb * kBlk * kBlk);
  oq_expand(params, nb, 1, Ti.data());  // kron of the factor inverses = T_b^-1
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b) {
      double wb[kBlk];
      for (int i = 0; i < kBlk; ++i) wb[i] = oq_load(w, dtype, r * ldw + b * kBlk + i);
      const double* Tb = Ti.data() + b * kBlk * kBlk;
      for (int j = 0; j < kBlk; ++j) {
        double acc = 0.0;
        for (int i = 0; i < kBlk; ++i) acc += wb[i] * Tb[i * kBlk + j];
        w_out[r * d + b * kBlk + j] = acc;
      }
    }
  return 0;
}

int oq_quantize_weights(const void* w, int dtype, int64_t rows, int64_t d, int64_t ldw,
                        const float* params, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds,
                        double* w_out, int nthreads) {
  if (!w || !params || !q || !s || bad_shape(rows, d, ldw) ||
      (dtype != OQ_BF16 && dtype != OQ_FP32) || ldq < d / 2 || lds < d / kBlk)
    return -1;
  int rc = 0;
  parallel_rows(rows, nthreads, [&](int64_t r0, int64_t r1) {
    const int64_t n = r1 - r0;
    std::vector<double> buf;
    double* y = w_out ? w_out + r0 * d : (buf.resize((size_t)n * d), buf.data());
    const uint8_t* base = (const uint8_t*)w + r0 * ldw * (dtype == OQ_BF16 ? 2 : 4);
    if (oq_weight_transform(base, dtype, n, d, ldw, params, y) != 0 ||
        oq_encode(y, n, d, q + r0 * ldq, ldq, s + r0 * lds, lds) != 0)
      rc = -1;
  });
  return rc;
}

}  // extern "C"

namespace {
// Signed order of codes: -6 < ... < -0.5 < -0 < +0 < 0.5 < ... < 6.
int code_order(int c) { return (c & 8) ? -(c & 7) - 1 : (c & 7); }
}  // namespace

extern "C" int oq_classify(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                           const double* y_o, int tol_mode, double tol_coef,
                           const uint8_t* q, int64_t ldq, const uint8_t* s, int64_t lds,
                           const float* y_c, int64_t ldy, double* stats) {
  if (!x || !y_o || !q || !s || !stats || bad_shape(rows, d, ldx) ||
      (tol_mode != 0 && tol_mode != 1) || ldq < d / 2 || lds < d / kBlk ||
      (y_c && ldy < d))
    return -1;
  for (int i = 0; i < 8; ++i) stats[i] = 0.0;
  stats[7] = -1.0;
  const int64_t nb = d / kBlk;
  for (int64_t t = 0; t < rows; ++t)
    for (int64_t b = 0; b < nb; ++b) {
      const double* yb = y_o + t * d + b * kBlk;
      double xmax = 0.0, amax = 0.0;
      for (int i = 0; i < kBlk; ++i) {
        xmax = std::max(xmax, std::fabs(oq_load(x, dtype, t * ldx + b * kBlk + i)));
        amax = std::max(amax, std::fabs(yb[i]));
      }
      const double norm = tol_mode == 0 ? xmax : amax;
      const double tol = tol_coef * norm;

      if (y_c)
        for (int i = 0; i < kBlk; ++i) {
          const double err = std::fabs((double)y_c[t * ldy + b * kBlk + i] - yb[i]);
          if (!(err <= tol)) stats[5] += 1;
          const double nerr = norm > 0 ? err / norm : err;
          if (!(nerr <= stats[6])) stats[6] = nerr;
        }

      const int e_o = oq_scale_exp(amax);
      const int s_c = s[t * lds + b];
      int e_use = e_o;
      bool scale_excused = false;
      if (s_c != e_o + 127) {
        const int e_lo = oq_scale_exp(std::max(0.0, amax - tol));
        const int e_hi = oq_scale_exp(amax + tol);
        const int e_c = s_c - 127;
        if (s_c != 0xFF && e_lo <= e_c && e_c <= e_hi) {
          scale_excused = true;
          e_use = e_c;
          stats[3] += 1;
        } else {
          stats[4] += 1;
          stats[2] += kBlk;
          if (stats[7] < 0) stats[7] = (double)(t * d + b * kBlk);
          continue;
        }
      }
      for (int i = 0; i < kBlk; ++i) {
        const uint8_t byte = q[t * ldq + b * (kBlk / 2) + i / 2];
        const int cand = (i & 1) ? (byte >> 4) : (byte & 0xF);
        const int ref = oq_e2m1_code(yb[i], e_use);
        bool ok = cand == ref;
        if (!ok) {
          const int lo = oq_e2m1_code(yb[i] - tol, e_use);
          const int hi = oq_e2m1_code(yb[i] + tol, e_use);
          ok = code_order(lo) <= code_order(cand) && code_order(cand) <= code_order(hi);
          if (ok) {
            stats[1] += 1;
            continue;
          }
          stats[2] += 1;
          if (stats[7] < 0) stats[7] = (double)(t * d + b * kBlk + i);
          continue;
        }
        if (scale_excused) stats[1] += 1;
        else stats[0] += 1;
      }
    }
  return 0;
}
