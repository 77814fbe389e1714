// Offline expansion of a mixed-radix side's learnable parameters into the
// blocks that the mixed-radix rotation kernels apply.
//
// HARP technical summary §2.1-2.2 ("HARP: Hadamard-Preconditioned Adaptive
// Rotation Processor for Extreme LLM Quantization", gist.science): stage t of
// the schedule applies one block per group, B = Q(theta) G_{b_t}, where
//   * G_b is the fixed base mixer: the normalised Sylvester Hadamard H_b/sqrt(b)
//     for powers of two, otherwise the orthogonal factor of the QR
//     factorisation of a fixed Gaussian matrix (R's diagonal made positive,
//     which makes the factor unique);
//   * Q is the learnable orthogonal part: a Givens rotation by phi for
//     b = 2, the Cayley map (I - A)(I + A)^-1 of a skew-symmetric A for
//     b > 2, so zero parameters give Q = I and B = G.
// Host code with no HIP dependency: float64 arithmetic, float32 result.
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <utility>
#include <vector>

#include "../../include/harp.h"

namespace {

bool pow2(int32_t v) { return v > 0 && (v & (v - 1)) == 0; }

// G = H_b / sqrt(b), H[i][j] = (-1)^popcount(i & j) (Sylvester's construction).
void sylvester(int b, std::vector<double>& G) {
  G.assign(static_cast<size_t>(b) * b, 0.0);
  const double s = 1.0 / std::sqrt(static_cast<double>(b));
  for (int i = 0; i < b; ++i)
    for (int j = 0; j < b; ++j)
      G[static_cast<size_t>(i) * b + j] = (__builtin_popcount(i & j) & 1) ? -s : s;
}

// Orthogonal factor of g = Q R (b x b, row-major) by Householder reflections,
// with the columns of Q negated where R's diagonal is negative, so that R
// has a positive diagonal.  False when g is rank-deficient (a zero on R's
// diagonal leaves the factor undetermined).
bool qr_positive(int b, const double* g, std::vector<double>& Q) {
  const size_t n = static_cast<size_t>(b);
  std::vector<double> A(g, g + n * n), v(n);
  Q.assign(n * n, 0.0);
  for (size_t i = 0; i < n; ++i) Q[i * n + i] = 1.0;
  for (size_t k = 0; k + 1 < n; ++k) {
    double norm2 = 0.0;
    for (size_t i = k; i < n; ++i) norm2 += A[i * n + k] * A[i * n + k];
    const double norm = std::sqrt(norm2);
    if (norm == 0.0) return false;
    // reflect column k onto alpha e_k, alpha of the sign opposite to the
    // pivot (no cancellation in v_k)
    const double alpha = A[k * n + k] >= 0.0 ? -norm : norm;
    for (size_t i = k; i < n; ++i) v[i] = A[i * n + k];
    v[k] -= alpha;
    double vv = 0.0;
    for (size_t i = k; i < n; ++i) vv += v[i] * v[i];
    if (vv == 0.0) continue;                 // column already alpha e_k
    // A <- H A on rows k.., H = I - 2 v v^T / (v^T v)
    for (size_t j = k; j < n; ++j) {
      double dot = 0.0;
      for (size_t i = k; i < n; ++i) dot += v[i] * A[i * n + j];
      const double f = 2.0 * dot / vv;
      for (size_t i = k; i < n; ++i) A[i * n + j] -= f * v[i];
    }
    // Q <- Q H on columns k..
    for (size_t r = 0; r < n; ++r) {
      double dot = 0.0;
      for (size_t i = k; i < n; ++i) dot += Q[r * n + i] * v[i];
      const double f = 2.0 * dot / vv;
      for (size_t i = k; i < n; ++i) Q[r * n + i] -= f * v[i];
    }
  }
  // g = Q R with R = A upper triangular; make R's diagonal positive
  for (size_t k = 0; k < n; ++k) {
    const double r = A[k * n + k];
    if (r == 0.0) return false;
    if (r < 0.0)
      for (size_t i = 0; i < n; ++i) Q[i * n + k] = -Q[i * n + k];
  }
  return true;
}

// Q = (I + A)^-1 (I - A) = (I - A)(I + A)^-1 (the two factors commute) for
// the skew-symmetric A whose upper triangle p holds A[r][c], r < c, row by
// row.  Solved by Gaussian elimination with partial pivoting on
// [I + A | I - A]; I + A is invertible for skew A (its eigenvalues are
// 1 + i lambda) and its singular values are at least 1.
void cayley(int b, const double* p, std::vector<double>& Q) {
  const size_t n = static_cast<size_t>(b), w = 2 * n;
  std::vector<double> M(n * w, 0.0);
  size_t k = 0;
  std::vector<double> A(n * n, 0.0);
  for (size_t r = 0; r < n; ++r)
    for (size_t c = r + 1; c < n; ++c, ++k) {
      A[r * n + c] = p[k];
      A[c * n + r] = -p[k];
    }
  for (size_t r = 0; r < n; ++r)
    for (size_t c = 0; c < n; ++c) {
      const double id = r == c ? 1.0 : 0.0;
      M[r * w + c] = id + A[r * n + c];
      M[r * w + n + c] = id - A[r * n + c];
    }
  for (size_t col = 0; col < n; ++col) {
    size_t piv = col;
    for (size_t r = col + 1; r < n; ++r)
      if (std::fabs(M[r * w + col]) > std::fabs(M[piv * w + col])) piv = r;
    if (piv != col)
      for (size_t c = 0; c < w; ++c) std::swap(M[col * w + c], M[piv * w + c]);
    const double d = M[col * w + col];
    for (size_t r = col + 1; r < n; ++r) {
      const double f = M[r * w + col] / d;
      if (f == 0.0) continue;
      for (size_t c = col; c < w; ++c) M[r * w + c] -= f * M[col * w + c];
    }
  }
  Q.assign(n * n, 0.0);
  for (size_t rr = n; rr-- > 0;) {
    for (size_t c = 0; c < n; ++c) {
      double s = M[rr * w + n + c];
      for (size_t j = rr + 1; j < n; ++j) s -= M[rr * w + j] * Q[j * n + c];
      Q[rr * n + c] = s / M[rr * w + rr];
    }
  }
}

}  // namespace

extern "C" harp_status harp_mixed_expand(int32_t n_stages, const int32_t* radix,
                                         const double* params, const double* gaussians,
                                         float* blocks) {
  if (radix == nullptr || params == nullptr || blocks == nullptr) return HARP_ERR_NULL;
  if (n_stages < 1 || n_stages > HARP_MAX_STAGES) return HARP_ERR_SHAPE;
  int64_t dim = 1;
  bool need_gauss = false;
  for (int t = 0; t < n_stages; ++t) {
    if (radix[t] > HARP_MAX_RADIX) return HARP_ERR_UNSUPPORTED;
    if (radix[t] < 2) return HARP_ERR_SHAPE;
    dim = dim * radix[t] > int64_t{HARP_MAX_MIXED_DIM} ? int64_t{HARP_MAX_MIXED_DIM} + 1
                                                         : dim * radix[t];
    need_gauss = need_gauss || !pow2(radix[t]);
  }
  if (dim > HARP_MAX_MIXED_DIM) return HARP_ERR_UNSUPPORTED;
  if (need_gauss && gaussians == nullptr) return HARP_ERR_NULL;
  // every parameter and Gaussian entry finite, every Gaussian of full rank
  const double* p = params;
  const double* g = gaussians;
  std::vector<std::vector<double>> mixers(static_cast<size_t>(n_stages));
  for (int t = 0; t < n_stages; ++t) {
    const int b = radix[t];
    const size_t np = static_cast<size_t>(dim / b) * (static_cast<size_t>(b) * (b - 1) / 2);
    for (size_t i = 0; i < np; ++i)
      if (!std::isfinite(p[i])) return HARP_ERR_SHAPE;
    p += np;
    if (pow2(b)) {
      sylvester(b, mixers[t]);
    } else {
      const size_t ng = static_cast<size_t>(b) * b;
      for (size_t i = 0; i < ng; ++i)
        if (!std::isfinite(g[i])) return HARP_ERR_SHAPE;
      if (!qr_positive(b, g, mixers[t])) return HARP_ERR_SHAPE;
      g += ng;
    }
  }
  // B = Q(theta) G per stage and group
  p = params;
  float* out = blocks;
  std::vector<double> Q;
  for (int t = 0; t < n_stages; ++t) {
    const size_t b = static_cast<size_t>(radix[t]);
    const size_t groups = static_cast<size_t>(dim) / b;
    const size_t np = b * (b - 1) / 2;
    const std::vector<double>& G = mixers[t];
    for (size_t c = 0; c < groups; ++c, p += np, out += b * b) {
      if (b == 2) {
        const double cs = std::cos(p[0]), sn = std::sin(p[0]);
        Q = {cs, -sn, sn, cs};
      } else {
        cayley(static_cast<int>(b), p, Q);
      }
      for (size_t r = 0; r < b; ++r)
        for (size_t j = 0; j < b; ++j) {
          double s = 0.0;
          for (size_t k = 0; k < b; ++k) s += Q[r * b + k] * G[k * b + j];
          out[r * b + j] = static_cast<float>(s);
        }
    }
  }
  return HARP_OK;
}
