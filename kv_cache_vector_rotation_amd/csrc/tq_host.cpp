// Host-only parts of libturboquant: status strings, the Lloyd-Max codebook
// builder, record geometry and the folding of the sketch with the rotation.
// No HIP runtime call is made from this file.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "tq_internal.h"
#include "turboquant.h"

namespace {

// ---------------------------------------------------------------------------
// Law of one coordinate of a uniformly random unit vector in R^d:
// density C_d (1 - y^2)^((d-3)/2) on [-1, 1]; y^2 ~ Beta(1/2, (d-1)/2).
// ([ZB] paragraph 2: after the random rotation each coordinate follows a Beta
// law.)
// ---------------------------------------------------------------------------

// Continued fraction of the regularized incomplete beta function (Euler's
// expansion), evaluated with the modified Lentz method:
//   I_x(a, b) = x^a (1 - x)^b / (a B(a, b)) / g,
//   g = 1 + d_1 / (1 + d_2 / (1 + d_3 / (1 + ...))),
//   d_{2k+1} = -(a + k)(a + b + k) x / ((a + 2k)(a + 2k + 1)),
//   d_{2k}   =  k (b - k) x / ((a + 2k - 1)(a + 2k)).
// It converges quickly for x < (a + 1) / (a + b + 2). Returns 1 / g.
double beta_cf(double a, double b, double x) {
  const double tiny = 1e-300;
  double f = 1.0, c = 1.0, dd = 0.0;
  for (int n = 1; n < 100000; ++n) {
    const int k = n / 2;
    const double num = (n % 2 == 1)
                           ? -(a + k) * (a + b + k) * x / ((a + 2.0 * k) * (a + 2.0 * k + 1.0))
                           : k * (b - k) * x / ((a + 2.0 * k - 1.0) * (a + 2.0 * k));
    dd = 1.0 + num * dd;
    if (std::fabs(dd) < tiny) dd = tiny;
    dd = 1.0 / dd;
    c = 1.0 + num / c;
    if (std::fabs(c) < tiny) c = tiny;
    const double delta = c * dd;
    f *= delta;
    if (std::fabs(delta - 1.0) < 1e-16) break;
  }
  return 1.0 / f;
}

// Regularized incomplete beta I_x(a, b), double precision.
double inc_beta(double a, double b, double x) {
  if (x <= 0.0) return 0.0;
  if (x >= 1.0) return 1.0;
  double lbeta = std::lgamma(a) + std::lgamma(b) - std::lgamma(a + b);
  double front = std::exp(a * std::log(x) + b * std::log1p(-x) - lbeta);
  if (x < (a + 1.0) / (a + b + 2.0)) return front * beta_cf(a, b, x) / a;
  return 1.0 - front * beta_cf(b, a, 1.0 - x) / b;
}

struct CoordLaw {
  int d;
  double norm;  // C_d
  explicit CoordLaw(int d_) : d(d_) {
    norm = std::exp(std::lgamma(d / 2.0) - std::lgamma((d - 1) / 2.0) - 0.5 * std::log(M_PI));
  }
  double cdf(double y) const {
    if (y <= -1.0) return 0.0;
    if (y >= 1.0) return 1.0;
    double i = inc_beta(0.5, (d - 1) / 2.0, y * y);
    return y >= 0 ? 0.5 + 0.5 * i : 0.5 - 0.5 * i;
  }
  // integral of y f(y) over [a, b]: C_d/(d-1) ((1-a^2)^((d-1)/2) - (1-b^2)^((d-1)/2))
  double first_moment(double a, double b) const {
    double e = (d - 1) / 2.0;
    auto p = [&](double y) {
      double u = 1.0 - y * y;
      if (u <= 0.0) return 0.0;
      return std::exp(e * std::log1p(-y * y));
    };
    return norm / (d - 1) * (p(a) - p(b));
  }
  double quantile(double u) const {  // bisection on the cdf
    double lo = -1.0, hi = 1.0;
    for (int i = 0; i < 200; ++i) {
      double mid = 0.5 * (lo + hi);
      if (cdf(mid) < u) lo = mid; else hi = mid;
    }
    return 0.5 * (lo + hi);
  }
};

}  // namespace

namespace tq {

bool layout_valid(const tq_layout* l) {
  if (!l) return false;
  if (l->mse_only != 0 && l->mse_only != 1) return false;
  if (l->norm_f16 != 0 && l->norm_f16 != 1) return false;
  if (l->d < 3 || l->d > 256) return false;
  if (l->n_groups != 1 && l->n_groups != 2) return false;
  int sum = 0;
  for (int g = 0; g < l->n_groups; ++g) {
    if (l->group_dim[g] < 3) return false;
    if (l->mse_bits[g] < 1 || l->mse_bits[g] > 4) return false;
    sum += l->group_dim[g];
  }
  return sum == l->d;
}

GroupGeom geometry(const tq_layout* l) {
  GroupGeom g{};
  g.n_groups = l->n_groups;
  int ch = 0, cw = 0, sw = 0, bcw = 0, bsw = 0, co = 0, bo = 0, bits = 0;
  for (int i = 0; i < l->n_groups; ++i) {
    int d = l->group_dim[i], m = l->mse_bits[i];
    g.dim[i] = d;
    g.bits[i] = m;
    g.ch_off[i] = ch;
    g.code_word_off[i] = cw;
    g.sign_word_off[i] = sw;
    g.blk_code_off[i] = bcw;
    g.blk_sign_off[i] = bsw;
    g.centroid_off[i] = co;
    g.boundary_off[i] = bo;
    ch += d;
    cw += (m * d + 31) / 32;
    sw += l->mse_only ? 0 : (d + 31) / 32;
    bcw += m * d;  // 32 rows * m * d bits / 32
    bsw += l->mse_only ? 0 : d;
    co += 1 << m;
    bo += (1 << m) - 1;
    bits += (l->mse_only ? m : m + 1) * d + (l->norm_f16 ? 32 : 64);
  }
  g.info.code_words = cw;
  g.info.sign_words = sw;
  g.info.norm_floats = 2 * l->n_groups;
  g.info.block_code_words = bcw;
  g.info.block_sign_words = bsw;
  g.info.record_bits = bits;
  return g;
}

bool quantizer_pointers_valid(const tq_quantizer* q) {
  if (!q) return false;
  const void* ps[5] = {q->rot, q->sketch, q->sketch_rot, q->centroids, q->boundaries};
  for (const void* p : ps) {
    if (!p) return false;
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return false;
  }
  return layout_valid(&q->layout);
}

}  // namespace tq

extern "C" {

int tq_abi_version(void) { return TQ_ABI_VERSION; }

const char* tq_status_string(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_ERR_INVALID: return "invalid argument";
    case TQ_ERR_UNSUPPORTED: return "unsupported shape for this build";
    case TQ_ERR_NOCONVERGE: return "Lloyd-Max did not converge";
    case TQ_ERR_WORKSPACE: return "workspace too small";
    case TQ_ERR_DEVICE: return "HIP device error";
    default: return "unknown status";
  }
}

// Lloyd-Max iteration on the coordinate law: boundaries are midpoints of
// neighbouring centroids; each centroid moves to the mean of its cell (closed
// first moment / cell mass); stop when no centroid moves more than tol; then
// enforce exact antisymmetry. mse = 1/d - sum_k P_k c_k^2 (centroid condition).
tq_status tq_build_codebook(int32_t d, int32_t mse_bits, int32_t max_iter, double tol,
                            double* centroids, double* boundaries, double* mse_per_coord) {
  if (d < 3 || mse_bits < 1 || mse_bits > 4 || !centroids || !boundaries || max_iter < 0 ||
      !(tol >= 0.0))
    return TQ_ERR_INVALID;
  const int L = 1 << mse_bits;
  if (max_iter == 0) max_iter = 200000;
  if (tol == 0.0) tol = 1e-13 / std::sqrt((double)d);
  CoordLaw law(d);
  std::vector<double> c(L), nc(L), t(L + 1), F(L + 1);
  for (int k = 0; k < L; ++k) c[k] = law.quantile((k + 0.5) / L);
  bool converged = false;
  for (int it = 0; it < max_iter; ++it) {
    t[0] = -1.0;
    t[L] = 1.0;
    for (int k = 1; k < L; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
    for (int k = 0; k <= L; ++k) F[k] = law.cdf(t[k]);
    double moved = 0.0;
    for (int k = 0; k < L; ++k) {
      nc[k] = law.first_moment(t[k], t[k + 1]) / (F[k + 1] - F[k]);
      moved = std::fmax(moved, std::fabs(nc[k] - c[k]));
    }
    c.swap(nc);
    if (moved < tol) {
      converged = true;
      break;
    }
  }
  if (!converged) return TQ_ERR_NOCONVERGE;
  for (int k = 0; k < L / 2; ++k) {
    double v = 0.5 * (c[L - 1 - k] - c[k]);
    c[k] = -v;
    c[L - 1 - k] = v;
  }
  for (int k = 0; k < L; ++k) centroids[k] = c[k];
  for (int k = 1; k < L; ++k) boundaries[k - 1] = 0.5 * (c[k - 1] + c[k]);
  if (mse_per_coord) {
    double s = 0.0;
    for (int k = 0; k < L; ++k) {
      double lo = k == 0 ? -1.0 : boundaries[k - 1];
      double hi = k == L - 1 ? 1.0 : boundaries[k];
      s += (law.cdf(hi) - law.cdf(lo)) * c[k] * c[k];
    }
    *mse_per_coord = 1.0 / d - s;
  }
  return TQ_OK;
}

tq_status tq_record_layout(const tq_layout* layout, tq_record_info* info) {
  if (!tq::layout_valid(layout) || !info) return TQ_ERR_INVALID;
  *info = tq::geometry(layout).info;
  return TQ_OK;
}

tq_status tq_fold_sketch(int32_t d, const float* rot, const float* sketch, float* sketch_rot) {
  if (d < 1 || d > 4096 || !rot || !sketch || !sketch_rot) return TQ_ERR_INVALID;
  // sketch_rot[i][j] = sum_k sketch[i][k] * rot[j][k]
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) {
      double s = 0.0;
      for (int k = 0; k < d; ++k) s += (double)sketch[i * d + k] * (double)rot[j * d + k];
      sketch_rot[i * d + j] = (float)s;
    }
  return TQ_OK;
}

}  // extern "C"
