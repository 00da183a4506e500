// Binary-coding quantization of an fp16 matrix: the planes b_i in {-1, +1} and
// group-wise fp16 scales alpha_i such that W ~ sum_i alpha_i * b_i (the format
// LUT-GEMM multiplies directly; Elamur card "LUT-GEMM -- paper by Park et al.
// (2022)", sections "Summary" and "Interesting ideas: Group size as a separate
// hyper-parameter"). The pages name the quantizer only by reference, so the
// method here is our own reading of the standard one:
//
//  * greedy: per (row, group), plane by plane, alpha_i is the mean absolute
//    residual (rounded to fp16), b_i its sign (zero counts as +1), and the
//    residual drops by alpha_i * b_i;
//  * alternating refinement (`iters` rounds after the greedy start): alpha is
//    refitted by least squares for the current planes (the q x q normal
//    equations, Gaussian elimination in row order without pivoting, then fp16
//    rounding; a singular or overflowing system keeps the previous alpha), and
//    each weight then takes the sign combination whose value is nearest (the
//    lowest combination index on ties, bit i of the index set = plane i is +1).
//
// Exactness: the inputs are fp16 (multiples of 2^-24), so every residual, every
// sum over a group and every candidate value is exact in binary64 as long as a
// group's absolute sums stay below 2^29; the only rounded steps are the
// divisions and the small elimination, done in the order written here.
#include <math.h>
#include <string.h>

#include "host_util.h"
#include "layout.h"
#include "lutgemm.h"

using namespace lutgemm;
using namespace lutgemm::host;

namespace {

constexpr int kMaxIters = 1000;

// One (row, group): w[0..g) in, b[i][k] (+1/-1) and alpha16[i] out. Returns the
// squared error of the result.
double quantize_group(const double* w, int g, int q, int iters, signed char* b, uint16_t* alpha16,
                      double* r) {
  // greedy
  for (int k = 0; k < g; ++k) r[k] = w[k];
  for (int i = 0; i < q; ++i) {
    double s = 0.0;
    for (int k = 0; k < g; ++k) s += fabs(r[k]);
    const uint16_t a = f64_to_f16_rne(s / g);
    const double av = f16_to_f64(a);
    alpha16[i] = a;
    for (int k = 0; k < g; ++k) {
      const signed char sg = r[k] >= 0.0 ? 1 : -1;
      b[i * g + k] = sg;
      r[k] -= sg > 0 ? av : -av;
    }
  }
  // alternating refinement
  double M[8][8], v[8], x[8];
  for (int it = 0; it < iters; ++it) {
    // least-squares scales for the current planes
    for (int i = 0; i < q; ++i) {
      for (int j = 0; j < q; ++j) {
        double m = 0.0;
        for (int k = 0; k < g; ++k) m += (double)(b[i * g + k] * b[j * g + k]);
        M[i][j] = m;
      }
      double t = 0.0;
      for (int k = 0; k < g; ++k) t += b[i * g + k] > 0 ? w[k] : -w[k];
      v[i] = t;
    }
    bool ok = true;
    for (int c = 0; c < q && ok; ++c) {
      const double piv = M[c][c];
      if (!(piv > 1e-9 * g)) {
        ok = false;
        break;
      }
      for (int rr = c + 1; rr < q; ++rr) {
        const double f = M[rr][c] / piv;
        for (int cc = c; cc < q; ++cc) M[rr][cc] -= f * M[c][cc];
        v[rr] -= f * v[c];
      }
    }
    if (ok) {
      for (int c = q - 1; c >= 0; --c) {
        double s = v[c];
        for (int cc = c + 1; cc < q; ++cc) s -= M[c][cc] * x[cc];
        x[c] = s / M[c][c];
      }
      uint16_t na[8];
      for (int i = 0; i < q; ++i) {
        na[i] = f64_to_f16_rne(x[i]);
        if (!f16_is_finite(na[i])) ok = false;
      }
      if (ok)
        for (int i = 0; i < q; ++i) alpha16[i] = na[i];
    }
    // nearest sign combination for every weight
    double val[256];
    const int nc = 1 << q;
    for (int c = 0; c < nc; ++c) {
      double s = 0.0;
      for (int i = 0; i < q; ++i) {
        const double a = f16_to_f64(alpha16[i]);
        s += ((c >> i) & 1) ? a : -a;
      }
      val[c] = s;
    }
    for (int k = 0; k < g; ++k) {
      int best = 0;
      double bd = fabs(w[k] - val[0]);
      for (int c = 1; c < nc; ++c) {
        const double d = fabs(w[k] - val[c]);
        if (d < bd) {
          bd = d;
          best = c;
        }
      }
      for (int i = 0; i < q; ++i) b[i * g + k] = ((best >> i) & 1) ? 1 : -1;
    }
  }
  double err = 0.0;
  for (int k = 0; k < g; ++k) {
    double s = 0.0;
    for (int i = 0; i < q; ++i) {
      const double a = f16_to_f64(alpha16[i]);
      s += b[i * g + k] > 0 ? a : -a;
    }
    err += (w[k] - s) * (w[k] - s);
  }
  return err;
}

}  // namespace

extern "C" int bcq_quantize(const lutgemm_shape* s, const uint16_t* w, int32_t iters,
                            uint8_t* bits, size_t bits_bytes, uint16_t* alpha, size_t alpha_count,
                            double* sq_error) {
  try {
    const int st = check_shape(s);
    if (st) return st;
    if (s->has_offset) return LUTGEMM_ERR_SHAPE;
    if (iters < 0 || iters > kMaxIters) return LUTGEMM_ERR_VALUE;
    const int64_t N = s->N, K = s->K, q = s->q, g = s->g;
    if (N == 0 || K == 0) {
      if (sq_error) *sq_error = 0.0;
      return LUTGEMM_OK;
    }
    if (!w || !bits || !alpha) return LUTGEMM_ERR_NULL;
    const size_t nb = (size_t)q * N * (K / 8), na = (size_t)q * N * (K / g);
    if (bits_bytes < nb || alpha_count < na) return LUTGEMM_ERR_BUFFER;
    for (size_t t = 0; t < (size_t)N * K; ++t)
      if (!f16_is_finite(w[t])) return LUTGEMM_ERR_VALUE;
    const int64_t G = K / g;
    std::vector<double> row_err((size_t)N, 0.0);
    parallel_for(N, [&](int64_t j0, int64_t j1) {
      std::vector<double> wg((size_t)g), r((size_t)g);
      std::vector<signed char> b((size_t)(q * g));
      for (int64_t j = j0; j < j1; ++j) {
        // this row's bytes are rewritten below, one group at a time
        for (int64_t i = 0; i < q; ++i) memset(bits + ((size_t)i * N + j) * (K / 8), 0, K / 8);
        double e = 0.0;
        for (int64_t t = 0; t < G; ++t) {
          for (int64_t k = 0; k < g; ++k) wg[k] = f16_to_f64(w[(size_t)j * K + t * g + k]);
          uint16_t a16[8];
          e += quantize_group(wg.data(), (int)g, (int)q, iters, b.data(), a16, r.data());
          for (int64_t i = 0; i < q; ++i) {
            alpha[((size_t)i * N + j) * G + t] = a16[i];
            uint8_t* row = bits + ((size_t)i * N + j) * (K / 8);
            for (int64_t k = 0; k < g; ++k)
              if (b[i * g + k] > 0) row[(t * g + k) >> 3] |= (uint8_t)(1u << ((t * g + k) & 7));
          }
        }
        row_err[(size_t)j] = e;
      }
    });
    if (sq_error) {
      double e = 0.0;
      for (double v : row_err) e += v;
      *sq_error = e;
    }
    return LUTGEMM_OK;
  } catch (...) {
    return LUTGEMM_ERR_INTERNAL;
  }
}
